// S4: gathered-row Q/K/V projection with a RoPE epilogue.
//
// QCFuse page, section 2.1.3 (Eq. 6-7): only the selected positions P (plus
// the query suffix) get fresh K/V under the current order and positions.
// KVBoost page, section 3.1 (Eq. 1): k = W_K x, v = W_V x; section 3.2 (Eq. 3):
// queries and keys carry the rotation of their position.
//
// bf16 path: Y[m, n] = sum_k X[row_src[m], k] W[n, k] on MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate); tiling and staging are
// described at the kernel.  Only the column tiles of the requested outputs
// (Q, K, V mask) are launched.
//
// fp32 path: a plain LDS-tiled FMA kernel (the fp32 workloads are small
// correctness shapes; MFMA is reserved for the bf16 contractions).
#include <climits>
#include <type_traits>

#include "../kvf_common.h"

namespace kvf {


struct GemmArgs {
  const void* x;
  int64_t x_rows;
  const int32_t* row_src;
  const int32_t* row_pos;
  int M;
  const void* w;
  int K;                    // hidden
  const float* rope_cos;
  const float* rope_sin;
  int rope_n;
  int d;
  int n_tiles[3];           // column tiles of the Q, K, V segments (0 if masked off)
  int seg_heads[3];         // heads of each segment
  int seg_w_row0[3];        // first weight row of each segment
  void* out[3];
  // split-K: blockIdx.z covers K range [z k_len, (z+1) k_len) and stores its
  // raw fp32 sums in partial (one tile-sized block per slice and output
  // tile); the last slice of an output tile to finish (tile_cnt counts
  // arrivals) adds the slices in order and finishes the rows.
  float* partial;
  int* tile_cnt;            // [row tiles x column tiles], zero between calls
  int k_len;
  // K/V destination rows: row m of K and V goes to row kv_row[m] of its
  // output (kv_rows rows; entries outside are skipped); nullptr: row m
  const int32_t* kv_row;
  int64_t kv_rows;
  int group_rows;           // row tiles per group of the dispatch order (xcd_tile)
};

// Output row of row m in segment seg (0 Q, 1 K, 2 V), or -1 to skip it.
__device__ __forceinline__ int64_t out_row(const GemmArgs& a, int seg, int m) {
  if (seg == 0 || !a.kv_row) return m;
  const int64_t r = a.kv_row[m];
  return (r >= 0 && r < a.kv_rows) ? r : -1;
}

// Row m is computed and stored only if its source row and (for Q/K) its
// position are inside the tables.
__device__ __forceinline__ bool row_ok(const GemmArgs& a, int m) {
  if (!a.row_src) return true;
  const int s = a.row_src[m];
  return s >= 0 && s < a.x_rows;
}

// Hardware hands workgroups to the 8 XCDs round-robin by linear id, and
// each XCD has its own L2.  Renumber so that XCD x runs one contiguous range
// of logical tiles, and order the logical tiles in groups of `gr` row tiles:
// within a group the row tile varies fastest, then the column tile.  The
// tiles an XCD holds at once then form a block of about gr rows by
// (resident tiles / gr) columns, whose X row panels and W column slabs are
// each fetched into that XCD's L2 once and shared by the block's tiles.
// gr = all row tiles gives whole column slabs (one W slab, every X panel).
__device__ __forceinline__ void xcd_tile(int gr, int& tx, int& ty, int& tz) {
  const int gx = gridDim.x, gy = gridDim.y;
  const int n = gx * gy * gridDim.z;
  const int b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int q = n >> 3, r = n & 7, x = b & 7;
  const int l = x * q + min(x, r) + (b >> 3);
  const int per_z = gx * gy;
  tz = l / per_z;
  const int lt = l - tz * per_z;
  const int grp = lt / (gr * gy);
  const int i = lt - grp * gr * gy;
  const int rows = min(gr, gx - grp * gr);   // the last group may be shorter
  ty = i / rows;
  tx = grp * gr + (i - ty * rows);
}

__device__ __forceinline__ int segment_of(const int (&n_tiles)[3], int& t) {
  int seg = 0;
  while (seg < 2 && t >= n_tiles[seg]) {
    t -= n_tiles[seg];
    ++seg;
  }
  return seg;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
// Workgroup tile BM x BN x 64 (BM a multiple of 32, BN 128 or 256, chosen per
// call so the tile count fills the chip in whole rounds); 4 waves in a
// WM x (4/WM) grid, each owning a (BM/WM) x (BN/(4/WM)) block of the tile
// as 32 x 32 MFMA accumulators.
// Operand tiles stream global -> LDS through the DMA path (16 bytes per lane,
// rows of X gathered through row_src by each lane's own source address) into
// a ring of 3-4 static stage buffers, so the next stages load while one
// computes.  Rows are 64 bf16 (8 chunks of 16 B) with chunks XOR-swizzled by
// row mod 8.  Few-row calls split K over blockIdx.z (see GemmArgs).
// Epilogue: 32 rows at a time go through LDS as fp32, where each thread
// takes 8 channels j.. of a head together with their RoPE partners j+d/2..,
// rotates them at the row's position and writes both as 16-byte bf16 stores.
// With K split, every slice stores its raw sums; the last slice of the tile
// to arrive reads all of them back in slice order and runs the epilogue.
constexpr int kBK = 64, kGThreads = 256;

template <int BM, int BN>
struct GemmTile {
  static constexpr int kA = BM * kBK;       // elements of an A stage
  static constexpr int kB = BN * kBK;       // elements of a B stage
  // stages in flight: as many as 160 KB of LDS holds, at most 4
  static constexpr int kStages =
      (kA + kB) * 2 * 4 <= 160 * 1024 ? 4 : ((kA + kB) * 2 * 3 <= 160 * 1024 ? 3 : 2);
  static_assert((kA + kB) * 2 * 2 <= 160 * 1024, "two stages must fit in LDS");
  // the epilogue stages fp32 results in the same memory, as many 32-row
  // blocks per round as fit
  static constexpr int kStageBytes = (kA + kB) * 2 * kStages;
  static constexpr int kEpRows = (160 * 1024 / (BN * 4)) / 32 * 32 < BM
                                     ? (160 * 1024 / (BN * 4)) / 32 * 32 : BM;
  static constexpr int kLdsBytes =
      kStageBytes > kEpRows * BN * 4 ? kStageBytes : kEpRows * BN * 4;
};

// Physical 16-B chunk of logical chunk `chunk` in LDS row `row` (rows of
// 128 B).  A 16-byte-per-lane read is served 16 lanes at a time across 64
// banks (256 B): the 16 rows a fragment read touches at once must cover both
// 128-B halves of the bank window with distinct chunks, hence row/2 in the
// XOR (rows r and r+8 differ in it, r and r+1 differ in the half).
__device__ __forceinline__ int gchunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ int gswz(int row, int chunk) {   // element offset of a 16-B chunk
  return row * kBK + (gchunk(row, chunk) << 3);
}

// One 16-byte-per-lane global -> LDS copy (the DMA path).  Issued from inline
// assembly so the copies are invisible to the compiler's wait-count tracking:
// their completion is awaited explicitly by dma_wait_barrier, which lets
// stages k+1.. stay in flight while stage k is read.  lds_base must be
// wave-uniform; lane l writes lds_base + 16 l.  The s_nop keeps one wait
// state between the M0 write and the copy that reads it.
__device__ __forceinline__ void dma16(const void* src, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src)
               : "memory");
}

// Wait until at most N of this wave's DMA copies are in flight, then meet
// the other waves: every wave's part of the stage has landed in LDS.  The
// workgroup fence of __syncthreads() would wait for all copies instead.
template <int N>
__device__ __forceinline__ void dma_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(N) : "memory");
}

// As dma_wait_barrier, after this wave's own LDS reads have completed: once
// every wave has passed it, the stage buffer those reads used may be
// overwritten.
template <int N>
__device__ __forceinline__ void lds_dma_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

template <int BM, int BN, int WM, bool SPLIT>
__global__ void __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_qkv_bf16_kernel(GemmArgs a) {
  constexpr int WN = 4 / WM;                // wave grid WM x WN
  constexpr int WR = BM / WM, WC = BN / WN; // rows and columns of one wave
  static_assert(WR % 32 == 0 && WC % 32 == 0, "wave block must be whole MFMA tiles");
  constexpr int MB = WR / 32;               // 32-row MFMA blocks per wave
  constexpr int NI = WC / 32;               // 32-column MFMA blocks per wave
  constexpr int AG = BM / 8;                // DMA groups (8 rows) of an A stage
  constexpr int BG = BN / 8;                // DMA groups of a B stage
  constexpr int AGW = AG / 4;               // A groups per wave (BM is a multiple of 32)
  constexpr int BGW = BG / 4;
  constexpr int PER = AGW + BGW;            // DMA instructions per wave per stage
  constexpr int NST = GemmTile<BM, BN>::kStages;
  constexpr int SA = GemmTile<BM, BN>::kA, SB = GemmTile<BM, BN>::kB;
  constexpr int ER = GemmTile<BM, BN>::kEpRows;
  // stage buffers A0..A(NST-1), B0..B(NST-1), reused by the epilogue
  __shared__ __attribute__((aligned(16))) unsigned char smem[GemmTile<BM, BN>::kLdsBytes];
  bf16_t* const a0s = reinterpret_cast<bf16_t*>(smem);
  bf16_t* const a1s = a0s + SA;
  bf16_t* const a2s = a0s + 2 * SA;
  bf16_t* const a3s = a0s + 3 * SA;
  bf16_t* const b0s = a0s + NST * SA;
  bf16_t* const b1s = b0s + SB;
  bf16_t* const b2s = b0s + 2 * SB;
  bf16_t* const b3s = b0s + 3 * SB;
  auto abuf = [&](auto i) -> bf16_t* {
    constexpr int I = decltype(i)::value;
    if constexpr (I == 0) return a0s; else if constexpr (I == 1) return a1s;
    else if constexpr (I == 2) return a2s; else return a3s;
  };
  auto bbuf = [&](auto i) -> bf16_t* {
    constexpr int I = decltype(i)::value;
    if constexpr (I == 0) return b0s; else if constexpr (I == 1) return b1s;
    else if constexpr (I == 2) return b2s; else return b3s;
  };

  int tx, t, kz;
  xcd_tile(a.group_rows, tx, t, kz);
  const int tile_id = tx + static_cast<int>(gridDim.x) * t;   // output tile (row tile fastest)
  const int seg = segment_of(a.n_tiles, t);
  const int n0 = t * BN;                    // first column inside the segment
  const int m0 = tx * BM;
  const int K = a.K;
  const int kz0 = kz * a.k_len;             // first k of this slice
  const bf16_t* X = static_cast<const bf16_t*>(a.x) + kz0;
  const bf16_t* W = static_cast<const bf16_t*>(a.w) + static_cast<int64_t>(a.seg_w_row0[seg] + n0) * K + kz0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w / WN, wc = w % WN;       // this wave's block of the tile
  // DMA slots: lane -> (row lane/8 of a group, physical chunk lane%8)
  const int drow = lane >> 3, dchunk = lane & 7;
  const bf16_t* asrc[AGW];
#pragma unroll
  for (int i = 0; i < AGW; ++i) {
    const int row = (w + 4 * i) * 8 + drow;
    const int m = m0 + row;
    int64_t src = 0;
    if (m < a.M) {
      src = a.row_src ? static_cast<int64_t>(a.row_src[m]) : m;
      if (src < 0 || src >= a.x_rows) src = 0;     // row skipped at the store
    }
    asrc[i] = X + src * K + (gchunk(row, dchunk) << 3);
  }
  const bf16_t* bsrc[BGW];
#pragma unroll
  for (int i = 0; i < BGW; ++i) {
    const int row = (w + 4 * i) * 8 + drow;
    bsrc[i] = W + static_cast<int64_t>(row) * K + (gchunk(row, dchunk) << 3);
  }
  auto dma_stage = [&](bf16_t* as, bf16_t* bs, int k0) {
#pragma unroll
    for (int i = 0; i < AGW; ++i) dma16(asrc[i] + k0, as + (w + 4 * i) * 8 * kBK);
#pragma unroll
    for (int i = 0; i < BGW; ++i) dma16(bsrc[i] + k0, bs + (w + 4 * i) * 8 * kBK);
  };
  // copies [i0, i1) of a stage (A copies first, then B)
  auto dma_part = [&](bf16_t* as, bf16_t* bs, int k0, auto i0c, auto i1c) {
    constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      if (i < AGW) dma16(asrc[i] + k0, as + (w + 4 * i) * 8 * kBK);
      else dma16(bsrc[i - AGW] + k0, bs + (w + 4 * (i - AGW)) * 8 * kBK);
    }
  };

  // The epilogue's rows (thread tid handles units tid + 256 i of each round;
  // a unit is 8 low channels of a head plus their partners in one row): read
  // their positions and validity now, off the epilogue's critical path.
  constexpr int UPR = BN / 16;                          // units per row
  constexpr int UPT = ER * UPR / kGThreads;             // units per thread per round
  static_assert(ER * UPR % kGThreads == 0, "whole units per thread");
  constexpr int ROUNDS = (BM + ER - 1) / ER;
  int epos[ROUNDS][UPT];
  int64_t erow[ROUNDS][UPT];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd)
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int m = m0 + rd * ER + (tid + kGThreads * i) / UPR;
      int pos = -1;                                     // -1: row not stored
      int64_t orow = -1;
      if (rd * ER + (tid + kGThreads * i) / UPR < BM && m < a.M && row_ok(a, m)) {
        pos = a.row_pos[m];
        if (seg < 2 && (pos < 0 || pos >= a.rope_n)) pos = -1;
        if (seg == 2) pos = 0;
        orow = out_row(a, seg, m);
        if (orow < 0) pos = -1;
      }
      epos[rd][i] = pos;
      erow[rd][i] = orow;
    }

  // operand read offsets (the swizzle depends on row mod 8 = lane mod 8)
  const int lr = lane & 31, hf = lane >> 5;
  int aoff[kBK / 16], boff[kBK / 16];
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    aoff[kk] = gswz(WR * wr + lr, 2 * kk + hf);   // + 32 mi rows
    boff[kk] = gswz(WC * wc + lr, 2 * kk + hf);   // + 32 ni rows
  }

  f32x16_t acc[MB][NI];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Operand fragments of k-step kk+1 are read while the MFMAs of kk run, and
  // across stages: the first fragments of stage k+1 are read before the last
  // MFMAs of stage k.
  constexpr int KK = kBK / 16;
  bf16x8_t af[2][MB], bfr[2][NI];
  auto load_frags = [&](const bf16_t* as, const bf16_t* bs, int slot, int kk) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      bfr[slot][ni] = *reinterpret_cast<const bf16x8_t*>(bs + ni * 32 * kBK + boff[kk]);
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
      af[slot][mi] = *reinterpret_cast<const bf16x8_t*>(as + mi * 32 * kBK + aoff[kk]);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][mi], bfr[slot][ni], acc[mi][ni], 0, 0, 0);
  };

  // Ring of NST stage buffers; stage k lives in buffer k % NST.  Once every
  // wave holds the fragments of stage k's last k-step, the waves meet (which
  // also means stage k+1 has landed) and buffer k % NST is free; its refill
  // with stage k+NST is issued during the first k-steps of stage k+1, a
  // few copies between MFMA groups, so the copy instructions never pile up
  // in the memory pipeline ahead of the MFMAs.
  const int nk = a.k_len / kBK;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  dma_stage(abuf(I0{}), bbuf(I0{}), 0);
  if (1 < nk) dma_stage(abuf(I1{}), bbuf(I1{}), kBK);
  if (NST > 2 && 2 < nk) dma_stage(abuf(I2{}), bbuf(I2{}), 2 * kBK);
  if (NST > 3 && 3 < nk) dma_stage(abuf(I3{}), bbuf(I3{}), 3 * kBK);
  // stage 0 landed: the copies of stages 1 .. min(NST, nk) - 1 may be pending
  {
    const int pend = min(NST, nk) - 1;
    if (pend >= 3) dma_wait_barrier<3 * PER>();
    else if (pend == 2) dma_wait_barrier<2 * PER>();
    else if (pend == 1) dma_wait_barrier<PER>();
    else dma_wait_barrier<0>();
  }
  load_frags(abuf(I0{}), bbuf(I0{}), 0, 0);
  constexpr int CPS = (PER + KK - 2) / (KK - 1);       // copies per k-step
  auto stage = [&](int k, auto cur, auto next, auto prev) {
    // buffer of stage k-1 gets stage k-1+NST
    const bool refill = k >= 1 && k - 1 + NST < nk;
    const int k0 = (k - 1 + NST) * kBK;
    auto step = [&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      load_frags(abuf(cur), bbuf(cur), (kk + 1) & 1, kk + 1);
      if (refill)
        dma_part(abuf(prev), bbuf(prev), k0, std::integral_constant<int, kk * CPS>{},
                 std::integral_constant<int, (kk + 1) * CPS < PER ? (kk + 1) * CPS : PER>{});
      mfmas(kk & 1);
    };
    step(I0{});
    if constexpr (KK > 2) step(I1{});
    if constexpr (KK > 3) step(I2{});
    static_assert(KK == 4, "k-steps per stage");
    // issue order: reads of k-step kk+1, then the MFMAs of kk
#pragma unroll
    for (int kk = 0; kk + 1 < KK; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x100, MB + NI, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MB * NI, 0);
    }
    if (k + 1 < nk) {
      // copies still allowed in flight: stages k+2 .. min(k+NST-1, nk-1)
      const int pend = min(NST - 2, nk - 2 - k);
      if (pend >= 2) lds_dma_wait_barrier<2 * PER>();
      else if (pend == 1) lds_dma_wait_barrier<PER>();
      else lds_dma_wait_barrier<0>();
    }
    // after the last stage these reads are unused (their buffer is settled:
    // no copy is in flight); one unconditional path keeps the compiler's
    // LDS wait counts exact for the MFMAs below
    load_frags(abuf(next), bbuf(next), 0, 0);
    mfmas((KK - 1) & 1);
    __builtin_amdgcn_sched_group_barrier(0x100, MB + NI, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MB * NI, 0);
  };
  for (int kt = 0; kt < nk; kt += NST) {
    if constexpr (NST == 4) {
      stage(kt, I0{}, I1{}, I3{});
      if (kt + 1 < nk) stage(kt + 1, I1{}, I2{}, I0{});
      if (kt + 2 < nk) stage(kt + 2, I2{}, I3{}, I1{});
      if (kt + 3 < nk) stage(kt + 3, I3{}, I0{}, I2{});
    } else if constexpr (NST == 2) {
      stage(kt, I0{}, I1{}, I1{});
      if (kt + 1 < nk) stage(kt + 1, I1{}, I0{}, I0{});
    } else {
      stage(kt, I0{}, I1{}, I2{});
      if (kt + 1 < nk) stage(kt + 1, I1{}, I2{}, I0{});
      if (kt + 2 < nk) stage(kt + 2, I2{}, I0{}, I1{});
    }
  }

  if constexpr (SPLIT) {
    // Raw slice sums in the thread's own order: slice z, output tile, then
    // per (32-row block, 32-column block, 4-row group) one 16-byte chunk per
    // thread, so every wave store or load is 1 KB contiguous.  Stored and
    // read with device-scope coherence (the slices run on different XCDs).
    constexpr int CH = MB * NI * 4;                  // chunks per thread
    const int64_t tiles = static_cast<int64_t>(gridDim.x) * gridDim.y;
    const __amdgpu_buffer_rsrc_t pr =
        handoff_rsrc(a.partial, static_cast<int64_t>(gridDim.z) * tiles * CH * kGThreads * 16);
    const uint32_t lane_off = static_cast<uint32_t>(tid) * 16;
    auto chunk_off = [&](int z, int c) -> uint32_t {    // uniform part: a scalar offset
      return static_cast<uint32_t>(((z * tiles + tile_id) * CH + c) * kGThreads * 16);
    };
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x4_t v = {acc[mi][ni][4 * rq], acc[mi][ni][4 * rq + 1], acc[mi][ni][4 * rq + 2],
                             acc[mi][ni][4 * rq + 3]};
          put_dev4(pr, lane_off, chunk_off(kz, (mi * NI + ni) * 4 + rq), v);
        }
    // (the stage buffers are idle: every copy has landed and been read)
    if (!arrive_last(a.tile_cnt + tile_id, static_cast<int>(gridDim.z), reinterpret_cast<int*>(smem)))
      return;
    // the last slice to arrive: the tile's sums over slices 0, 1, .. in order
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
    for (int z = 0; z < static_cast<int>(gridDim.z); ++z) {
#pragma unroll
      for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const f32x4_t v = get_dev4(pr, lane_off, chunk_off(z, (mi * NI + ni) * 4 + rq));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mi][ni][4 * rq + e] += v[e];
          }
    }
  }
  __syncthreads();

  // epilogue through LDS, ER rows per round as fp32 (16-B chunks swizzled)
  float* ep = reinterpret_cast<float*>(smem);
  auto eidx = [](int row, int col) {
    return row * BN + ((((col >> 2) ^ (row & 31))) << 2) + (col & 3);
  };
  const bool rope = seg < 2;
  const int d = a.d, half = d >> 1;
  const int ld = a.seg_heads[seg] * d;
  bf16_t* out = static_cast<bf16_t*>(a.out[seg]);
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    if (m0 + rd * ER >= a.M) break;          // block-uniform
    // rows [rd ER, rd ER + ER) of the tile: this wave's 32-row blocks in them
#pragma unroll
    for (int mi = 0; mi < MB; ++mi) {
      const int trow = WR * wr + 32 * mi;    // first tile row of the block
      if (trow < rd * ER || trow >= rd * ER + ER) continue;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = trow - rd * ER + 8 * (r >> 2) + 4 * hf + (r & 3);
          ep[eidx(row, WC * wc + 32 * ni + lr)] = acc[mi][ni][r];
        }
    }
    __syncthreads();
    // read every unit's rope factors first, then rotate and store
    float lo[UPT][8], hi[UPT][8], cs[UPT][8], sn[UPT][8];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + kGThreads * i;
      const int row = u / UPR, p = u % UPR;
      const int head = p / (half / 8), j0 = (p % (half / 8)) * 8;
      const int cl = head * d + j0, ch = cl + half;
      const int pos = epos[rd][i];
      if (rope && pos >= 0) {
        Elem<float>::load8(a.rope_cos + static_cast<int64_t>(pos) * half + j0, cs[i]);
        Elem<float>::load8(a.rope_sin + static_cast<int64_t>(pos) * half + j0, sn[i]);
      }
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        const float4 l4 = *reinterpret_cast<const float4*>(&ep[eidx(row, cl + 4 * hp)]);
        const float4 h4 = *reinterpret_cast<const float4*>(&ep[eidx(row, ch + 4 * hp)]);
        lo[i][4 * hp] = l4.x; lo[i][4 * hp + 1] = l4.y; lo[i][4 * hp + 2] = l4.z; lo[i][4 * hp + 3] = l4.w;
        hi[i][4 * hp] = h4.x; hi[i][4 * hp + 1] = h4.y; hi[i][4 * hp + 2] = h4.z; hi[i][4 * hp + 3] = h4.w;
      }
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int p = (tid + kGThreads * i) % UPR;
      const int head = p / (half / 8), j0 = (p % (half / 8)) * 8;
      const int cl = head * d + j0, ch = cl + half;
      const int pos = epos[rd][i];
      if (pos < 0) continue;
      if (rope) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = lo[i][e], y = hi[i][e];
          lo[i][e] = x * cs[i][e] - y * sn[i][e];
          hi[i][e] = y * cs[i][e] + x * sn[i][e];
        }
      }
      bf16_t* orow = out + erow[rd][i] * ld + n0;
      Elem<bf16_t>::store8(orow + cl, lo[i]);
      Elem<bf16_t>::store8(orow + ch, hi[i]);
    }
    if (rd + 1 < ROUNDS) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: tile of 32 rows x 64 RoPE pairs (128 columns), BK = 32
// ---------------------------------------------------------------------------
constexpr int kFM = 32, kFP = 64, kFK = 32;

__global__ void __launch_bounds__(256) gemm_qkv_f32_kernel(GemmArgs a, int pair_tiles0,
                                                           int pair_tiles1, int pair_tiles2) {
  __shared__ float Xs[kFM][kFK + 1];
  __shared__ float Wlo[kFP][kFK + 1];
  __shared__ float Whi[kFP][kFK + 1];
  int t = blockIdx.y;
  const int pt[3] = {pair_tiles0, pair_tiles1, pair_tiles2};
  int seg = 0;
  while (seg < 2 && t >= pt[seg]) {
    t -= pt[seg];
    ++seg;
  }
  const int d = a.d, half = d >> 1;
  const int heads = a.seg_heads[seg];
  const int K = a.K;
  const float* X = static_cast<const float*>(a.x);
  const float* W = static_cast<const float*>(a.w) + static_cast<int64_t>(a.seg_w_row0[seg]) * K;
  const int tid = threadIdx.x;
  const int p = tid & 63, rg = tid >> 6;
  const int P = t * kFP + p;                     // pair index in the segment
  const int head = P / half, j = P % half;
  const bool pvalid = head < heads;
  const int m0 = blockIdx.x * kFM;

  float alo[8], ahi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) alo[i] = ahi[i] = 0.f;

  for (int k0 = 0; k0 < K; k0 += kFK) {
    // X tile: 32 x 32
    for (int e = tid; e < kFM * kFK; e += 256) {
      const int rr = e / kFK, kk = e % kFK;
      const int m = m0 + rr;
      float v = 0.f;
      if (m < a.M) {
        const int64_t src = a.row_src ? a.row_src[m] : m;
        if (src >= 0 && src < a.x_rows) v = X[src * K + k0 + kk];
      }
      Xs[rr][kk] = v;
    }
    // W tiles: low and high halves of 64 pairs
    for (int e = tid; e < kFP * kFK; e += 256) {
      const int pp = e / kFK, kk = e % kFK;
      const int PP = t * kFP + pp;
      const int hh = PP / half, jj = PP % half;
      float lo = 0.f, hi = 0.f;
      if (hh < heads) {
        lo = W[static_cast<int64_t>(hh * d + jj) * K + k0 + kk];
        hi = W[static_cast<int64_t>(hh * d + half + jj) * K + k0 + kk];
      }
      Wlo[pp][kk] = lo;
      Whi[pp][kk] = hi;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kFK; ++kk) {
      const float wl = Wlo[p][kk], wh = Whi[p][kk];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xv = Xs[rg + 4 * i][kk];
        alo[i] = fmaf(xv, wl, alo[i]);
        ahi[i] = fmaf(xv, wh, ahi[i]);
      }
    }
    __syncthreads();
  }
  if (!pvalid) return;
  float* out = static_cast<float*>(a.out[seg]);
  const int ld = heads * d;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + rg + 4 * i;
    if (row >= a.M || !row_ok(a, row)) continue;
    float lo = alo[i], hi = ahi[i];
    if (seg < 2) {
      const int pos = a.row_pos[row];
      if (pos < 0 || pos >= a.rope_n) continue;
      const float c = a.rope_cos[static_cast<int64_t>(pos) * half + j];
      const float s = a.rope_sin[static_cast<int64_t>(pos) * half + j];
      const float l2 = lo * c - hi * s;
      hi = hi * c + lo * s;
      lo = l2;
    }
    const int64_t dst = out_row(a, seg, row);
    if (dst < 0) continue;
    out[dst * ld + head * d + j] = lo;
    out[dst * ld + head * d + half + j] = hi;
  }
}

namespace {

struct Bf16Plan {
  int bm, bn, wm, splits;
  int n_tiles[3];           // column tiles per segment at bn
};

// Tile shape of a bf16 call.  Column tile 256 when every requested segment
// is a multiple of it; row-tile height the candidate whose tiles fill 256 CUs
// with the least per-CU work (rounds x tile area, ties to the larger tile).
// A call with too few tiles for half the chip (few rows) takes 64 or
// 128 x 128 tiles instead and may split K into 2^j slices of >= 256, added
// by the last slice of each output tile to finish.  The slice count is the
// one with the least estimated time: these tiles hold one workgroup per CU,
// so the workgroups run in ceil(n / 256) rounds, each a K loop of hidden / sp
// plus a fixed cost (prologue and epilogue, about kRoundFixedK k-columns of
// loop), plus one hand-off when K is split.  (Counting only how close the
// workgroups come to one per CU put the 70B-shaped 256-row probe at 320
// workgroups, two rounds of half-length loops: 102 us.)
constexpr int64_t kRoundFixedK = 1024;   // a round's fixed cost in k-columns of loop (about 5 us)
constexpr int64_t kHandoffK = 1024;      // storing, counting and re-reading the slices
Bf16Plan plan_bf16(const kvf_layer_desc& L, int M, uint32_t mask) {
  const int heads[3] = {L.n_q_heads, L.n_kv_heads, L.n_kv_heads};
  const uint32_t bits[3] = {KVF_OUT_Q, KVF_OUT_K, KVF_OUT_V};
  auto tiles = [&](int bn, int* per) {
    int total = 0;
    for (int s = 0; s < 3; ++s) {
      const int cols = heads[s] * L.head_dim;
      const int t = (mask & bits[s]) ? cols / bn : 0;
      if (per) per[s] = t;
      total += t;
    }
    return total;
  };
  Bf16Plan p{128, 256, 1, 1, {0, 0, 0}};
  for (int s = 0; s < 3; ++s)
    if ((mask & bits[s]) && (heads[s] * L.head_dim) % 256 != 0) p.bn = 128;
  const int total = tiles(p.bn, p.n_tiles);
  int64_t best_cost = INT64_MAX;
  for (int bm : {256, 192, 160, 128}) {
    if (p.bn == 256 && bm > 160) continue;      // fewer than 3 stages fit in LDS
    const int64_t blocks = static_cast<int64_t>(ceil_div(M, bm)) * total;
    const int64_t cost = (blocks + 255) / 256 * bm;
    if (cost < best_cost) {
      best_cost = cost;
      p.bm = bm;
    }
  }
  if (static_cast<int64_t>(ceil_div(M, p.bm)) * total >= 128) return p;
  Bf16Plan q{M <= 64 ? 64 : 128, 128, 1, 1, {0, 0, 0}};
  const int64_t base = static_cast<int64_t>(ceil_div(M, q.bm)) * tiles(128, q.n_tiles);
  int64_t best_time = INT64_MAX;
  for (int sp = 1; sp == 1 || (L.hidden % (sp * kBK) == 0 && L.hidden / sp >= 256); sp *= 2) {
    const int64_t rounds = (base * sp + kCUs - 1) / kCUs;
    const int64_t cost = rounds * (L.hidden / sp + kRoundFixedK) + (sp > 1 ? kHandoffK : 0);
    if (cost < best_time) {
      best_time = cost;
      q.splits = sp;
    }
  }
  return q;                                // smaller tiles, split or not: more workgroups than p
}

// Rows per group of the dispatch order (xcd_tile).  The tiles one XCD holds
// at once (one workgroup per CU, at most its share of the grid: `resident`
// consecutive logical tiles) span some row tiles and column tiles, whose
// operands it fetches: bm rows of X per row tile and bn rows of W per column
// tile, per k.  Pick the gr with the fewest, ties to the taller group.
int group_rows(int nrow, int ncol, int bm, int bn) {
  const int64_t tiles = static_cast<int64_t>(nrow) * ncol;
  const int resident = static_cast<int>(std::min<int64_t>(kCUs / 8, (tiles + 7) / 8));
  int best = nrow;
  int64_t best_cost = INT64_MAX;
  for (int gr = nrow; gr >= 1; --gr) {
    int rows, cols;
    if (resident <= gr) {                       // part of one column of a group
      rows = resident;
      cols = 1;
    } else if (resident <= gr * ncol) {         // gr rows, a few columns
      rows = gr;
      cols = ceil_div(resident, gr);
    } else {                                    // whole groups: every column
      rows = ceil_div(resident, ncol);
      cols = ncol;
    }
    const int64_t cost = static_cast<int64_t>(rows) * bm + static_cast<int64_t>(cols) * bn;
    if (cost < best_cost) {
      best_cost = cost;
      best = gr;
    }
  }
  return best;
}

}  // namespace

// Split-K workspace: kSplitCounterBytes of arrival counters (one int per
// output tile, zero between calls), then the slices' partial sums.  The
// counters sit at a fixed offset so that calls of any shape can share one
// workspace without their partial sums landing on another call's counters.
constexpr int kSplitCounterBytes = 4096;

size_t recompute_workspace(const kvf_layer_desc& L, int M, uint32_t mask) {
  if (L.dtype != KVF_BF16 || M <= 0 || mask == 0) return 0;
  const Bf16Plan p = plan_bf16(L, M, mask);
  if (p.splits == 1) return 0;
  const int64_t tiles = static_cast<int64_t>(ceil_div(M, p.bm)) * (p.n_tiles[0] + p.n_tiles[1] + p.n_tiles[2]);
  return kSplitCounterBytes + static_cast<size_t>(p.splits) * tiles * p.bm * p.bn * sizeof(float);
}

hipError_t launch_recompute(const kvf_layer_desc& L, const void* x, int64_t x_rows,
                            const int32_t* row_src, const int32_t* row_pos, int M, const void* w,
                            uint32_t mask, const float* rc, const float* rs, int rope_n, void* q,
                            void* k, void* v, const int32_t* kv_row, int64_t kv_rows, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  GemmArgs a{};
  a.kv_row = kv_row;
  a.kv_rows = kv_rows;
  a.x = x;
  a.x_rows = x_rows;
  a.row_src = row_src;
  a.row_pos = row_pos;
  a.M = M;
  a.w = w;
  a.K = L.hidden;
  a.k_len = L.hidden;
  a.rope_cos = rc;
  a.rope_sin = rs;
  a.rope_n = rope_n;
  a.d = L.head_dim;
  const int heads[3] = {L.n_q_heads, L.n_kv_heads, L.n_kv_heads};
  const uint32_t bits[3] = {KVF_OUT_Q, KVF_OUT_K, KVF_OUT_V};
  void* outs[3] = {q, k, v};
  int row0 = 0;
  for (int s = 0; s < 3; ++s) {
    a.seg_heads[s] = heads[s];
    a.seg_w_row0[s] = row0;
    a.out[s] = outs[s];
    row0 += heads[s] * L.head_dim;
  }
  if (L.dtype == KVF_BF16) {
    for (int s = 0; s < 3; ++s)
      if ((heads[s] * L.head_dim) % 128 != 0) return hipErrorInvalidValue;  // rejected earlier
    if (L.hidden % kBK != 0) return hipErrorInvalidValue;
    const Bf16Plan p = plan_bf16(L, M, mask);
    int total = 0;
    for (int s = 0; s < 3; ++s) {
      a.n_tiles[s] = p.n_tiles[s];
      total += p.n_tiles[s];
    }
    if (total == 0 || total > 65535) return hipErrorInvalidValue;
    if (p.splits > 1) {
      if (ws == nullptr || ws_bytes < recompute_workspace(L, M, mask)) return hipErrorInvalidValue;
      if (static_cast<int64_t>(ceil_div(M, p.bm)) * total * static_cast<int64_t>(sizeof(int)) >
          kSplitCounterBytes)
        return hipErrorInvalidValue;                // the plan splits small calls only
      a.tile_cnt = static_cast<int*>(ws);
      a.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + kSplitCounterBytes);
      a.k_len = L.hidden / p.splits;
    }
    const dim3 grid(ceil_div(M, p.bm), total, p.splits);
    a.group_rows = group_rows(static_cast<int>(grid.x), total, p.bm, p.bn);
    bool launched = false;
    const bool split = p.splits > 1;
#define KVF_GEMM_CASE(BM_, BN_, WM_, SPLIT_)                                                  \
  if (!launched && p.bm == BM_ && p.bn == BN_ && p.wm == WM_ && split == SPLIT_) {            \
    hipLaunchKernelGGL((gemm_qkv_bf16_kernel<BM_, BN_, WM_, SPLIT_>), grid, dim3(kGThreads), 0, \
                       st, a);                                                                \
    launched = true;                                                                          \
  }
    KVF_GEMM_CASE(256, 128, 1, false)
    KVF_GEMM_CASE(192, 128, 1, false)
    KVF_GEMM_CASE(160, 128, 1, false)
    KVF_GEMM_CASE(128, 128, 1, false)
    KVF_GEMM_CASE(64, 128, 1, false)
    KVF_GEMM_CASE(160, 256, 1, false)
    KVF_GEMM_CASE(128, 256, 1, false)
    KVF_GEMM_CASE(128, 128, 1, true)     // the few-row plans that split K
    KVF_GEMM_CASE(64, 128, 1, true)
#undef KVF_GEMM_CASE
    if (!launched) return hipErrorInvalidValue;
  } else {
    int pt[3], total = 0;
    for (int s = 0; s < 3; ++s) {
      pt[s] = (mask & bits[s]) ? ceil_div(heads[s] * (L.head_dim / 2), kFP) : 0;
      total += pt[s];
    }
    if (L.hidden % kFK != 0 || total == 0 || total > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_qkv_f32_kernel, dim3(ceil_div(M, kFM), total), dim3(256), 0, st, a,
                       pt[0], pt[1], pt[2]);
  }
  return hipGetLastError();
}

}  // namespace kvf
