// S6: causal attention of the recomputed (sparse) query rows over the fused
// cache, and S2 query-to-context attention mass.
//
// Attention: QCFuse page, section 2.1.3 - a recomputed token at position p
// reads prefix positions j <= p of the fused cache; KVBoost page, section
// 3.1, Eq. 2 - softmax(q K^T / sqrt(d)) V over positions <= t.
// Attention mass: QCFuse page, section 3.2.1, Eq. 9-10 - the mass that the
// query tokens' attention puts on each context position, summed over query
// tokens and heads (one layer here).
//
// bf16 path (MFMA v_mfma_f32_32x32x16_bf16, fp32 softmax):
//  * A workgroup owns one kv head and 128 query vectors: R rows x G query
//    heads of that kv head (grouped-query packing), so every K/V tile staged
//    in LDS serves all G heads.  Workgroups are ordered kv-head-fastest:
//    consecutive workgroups land on different XCDs, so with 8 kv heads each
//    XCD's L2 holds a single head's K/V.  Row tiles run longest-first.
//  * Scores are computed transposed, S^T = K Q^T (keys on the MFMA rows), so
//    each lane holds one query vector's scores and the online-softmax max/sum
//    are lane-local plus one cross-half shuffle.  The probabilities then feed
//    O^T += V^T P^T directly from registers; the V operand comes from the
//    row-major V tile through transposing LDS reads (ds_read_b64_tr_b16).
//  * The causal mask uses each row's own position; keys beyond the tile's
//    last position are never loaded.
// The mass score (see the section below) takes per-chunk softmax statistics
// of the query rows, combines them into log-sum-exps, sums the normalised
// probabilities per key in a second MFMA pass and adds the kv heads in a
// fixed order, so the result is deterministic.
//
// Int8-resident fused cache (KVBoost page, section 4.5, Eq. 7 held by the
// fused cache; section 7.3: half the bytes of a 16-bit cache): the same
// kernel reads the 8-bit codes and each row's (min, scale), once per
// workgroup per tile on the way into LDS, and runs the fp16 MFMA
// (v_mfma_f32_32x32x16_f16) with queries and probabilities in fp16.
//  * Keys stay exact: the tile holds 1024 + code (an fp16 integer, built by
//    byte permutes), so the MFMA gives q . (1024 + c) exactly up to fp32
//    summation, and each key's affine map - scale and min - 1024 scale times
//    the query's channel sum - is applied to the fp32 scores.  (Rounding the
//    decoded keys to fp16 instead costs up to 2.2e-2 of an output vector on
//    peaked rows, the whole error budget.)
//  * Values are decoded to fp16 (min + code * scale, one rounding), whose
//    error averages out over the keys a row attends to.
//
// fp32 path: one wave per (row, head) with lane-parallel keys; used by the
// small fp32 workloads only.
#include <mutex>
#include <type_traits>

#include "../kvf_common.h"

namespace kvf {

constexpr int kAQ = 128;         // query vectors per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  BatchArgs b;
  int qrow0[KVF_MAX_REQ];        // first q row of each request in the q buffer
  int nrows[KVF_MAX_REQ];        // q rows of each request
  int pos0[KVF_MAX_REQ];         // position of the first row when q_pos is NULL
  int orow0[KVF_MAX_REQ];        // first output row of each request
  int cu_tiles[KVF_MAX_REQ + 1]; // row-tile prefix
  int total_tiles;
  int fold_from;                 // dispatch slots at or past this run smallest-first
  int interleave;                // > 0: requests of equal shape, interleaved in groups of this many
  int parts;                     // > 1: long row tiles split their keys over up to this many workgroups
  int split_min;                 // key tiles from which a row tile is split
  float* ws_part;                // [tiles * Hkv, parts, 16-byte chunks, threads]
  int* ws_cnt;                   // [tiles * Hkv] arrivals (workspace offset 0); zero between calls
  int rows_per_tile;             // R
  const void* q;
  const int32_t* q_pos;
  const void* k;                 // bf16 [rows, Hkv, d], or 8-bit codes (int8-resident)
  const void* v;
  const float* k_stats;          // int8-resident: [rows, Hkv, 2] (min, scale)
  const float* v_stats;
  void* out;                     // [out rows, Hq, d]
  float* lse;                    // [out rows, Hq] natural log (attention mode)
  float* part_m;                 // [splits, out rows, Hq] log2 domain (statistics mode)
  float* part_l;
  int64_t plane;                 // rows * Hq: stride between split planes
  int n_splits;
  int split_keys;                // keys per split (a multiple of the key tile)
  int hq, hkv, G;
  float scale_log2;
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
// A workgroup owns 128 query vectors; each of its waves owns kQB blocks of
// 32 of them (every K or V fragment read from LDS feeds kQB MFMAs).  Two
// workgroups share a CU (64 KB of LDS each), so their waves interleave on
// every SIMD without sharing barriers, and each wave accumulates the next
// key block's scores while this block's softmax runs.
//
// Keys advance in tiles of 64 (two 32-key blocks).  K and V tiles are copied
// global -> LDS by the DMA path (global_load_lds, 16 bytes per lane) into two
// K buffers and two V buffers, each a distinct static array so the compiler
// can tell the outstanding copies apart.  Per tile t, with barriers A and B:
//   A: V_t has landed; all waves are done with V_{t-1}  -> copy V_{t+1}
//      S(t, block 1) from K_t, overlapped with softmax(t, block 0)
//      O += P(t, block 0) V_t
//   B: K_{t+1} has landed; all waves are done with K_t  -> copy K_{t+2}
//      S(t+1, block 0) from K_{t+1}, overlapped with softmax(t, block 1)
//      O += P(t, block 1) V_t
// so every copy has a whole tile of compute to land.  Tiles are row-major
// with the 16-byte chunks of row r XOR-swizzled (chunk_xor): the key-row reads
// of the score MFMA and the transposing reads of V (ds_read_b64_tr_b16, one
// 4-key x 4-channel transpose per 16 lanes) hit distinct banks.
constexpr int kAT = 64;          // keys per tile (two 32-key blocks)
constexpr int kQB = 1;           // 32-vector query blocks per wave
constexpr int kAWaves = 4 / kQB; // 128 query vectors per workgroup
constexpr int kAThreads = 64 * kAWaves;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
// Word 3 of a gfx9-family buffer descriptor for raw byte addressing
// (stride 0): 32-bit data format, no swizzle; accesses at or past the
// descriptor's byte range read as zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Buffer descriptor over `bytes` bytes at `base` (wave-uniform values).
__device__ __forceinline__ u32x4_t buffer_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32) & 0xffffu);   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bytes));
  r[3] = kBufferRsrcWord3;
  return r;
}

// One 16-byte-per-lane buffer -> LDS copy (lane l writes LDS byte address
// lds + 16 l; lds wave-uniform; bytes past the descriptor's range land as
// zeros).
// Issued from inline assembly so that the compiler's wait-count tracking
// does not see it: it cannot tell which LDS buffer a copy writes, and would
// otherwise wait for every copy in flight before the next LDS read, that is
// half a tile after the copy was issued.  Completion is awaited explicitly
// by copies_landed_barrier.  The s_nop keeps one wait state between the M0
// write and the copy that reads it.
__device__ __forceinline__ void buffer_copy16(const u32x4_t& rsrc, int voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voff), "s"(rsrc) : "memory");
}

// XOR applied to the 16-byte chunk index of tile row `row`.  LDS serves a
// wide read over 64 banks (256 B) per cycle: 16 lanes of a 16-byte read or
// 32 lanes of an 8-byte one.
//  D = 128 (256-B rows, each row spans all banks): the 16 rows of a key read
//    need 16 distinct chunks, and the V transpose reads 4 consecutive rows x 4
//    adjacent chunks at once, so rows 0..3 must move the chunk into different
//    groups of 4: a rotation of the row's low 4 bits, (r & 3) << 2 | (r >> 2) & 3.
//  D = 64 (128-B rows, two rows per bank window): the same conditions apply
//    to row pairs, on bits 1..3 of the row.
template <int D>
__device__ __forceinline__ int chunk_xor(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  }
}

// Workgroup barrier after this wave's tile copies older than the newest N
// have landed (vmcnt counts only those copies here) and its LDS reads have
// returned.  One asm statement with a memory clobber, so the compiler moves
// no LDS access across the barrier.
template <int N>
__device__ __forceinline__ void copies_landed_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Q8: K/V are 8-bit codes with per-row statistics (int8-resident cache).
// Their tiles are not copied by DMA but loaded into registers a tile ahead
// (thread t: key row t / 4 of the tile, the 8-code pieces (t % 4) + 4 i),
// dequantised after the barrier that frees their LDS buffer and written as
// fp16; the piece order makes each 16-lane group of a write cover all 64
// banks.
template <int D, bool Q8>
__global__ void __launch_bounds__(kAThreads) __attribute__((amdgpu_waves_per_eu(2 / kQB, 2 / kQB)))
attn_mfma_kernel(AttnArgs a) {
  using OpT = std::conditional_t<Q8, f16x8_t, bf16x8_t>;   // MFMA operand (8 values)
  constexpr int KS = D / 16;       // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;       // 32-channel output blocks
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;    // rows per DMA instruction (64 lanes x 16 B)
  constexpr int NDMA = kAT / RPI / kAWaves;   // DMA instructions per wave per tile and tensor
  constexpr int TILE = kAT * D;
  static_assert(NDMA >= 1 && NDMA * RPI * kAWaves == kAT, "tile copy split");
  // the two K and two V tile buffers, one array so that every copy's LDS
  // address is one scalar base plus a constant
  __shared__ __attribute__((aligned(16))) bf16_t kvs[4 * TILE];
  bf16_t* const k0s = kvs;
  bf16_t* const k1s = kvs + TILE;
  bf16_t* const v0s = kvs + 2 * TILE;
  bf16_t* const v1s = kvs + 3 * TILE;
  __shared__ int s_pos[2];
  __shared__ int s_wpos[2 * kAWaves];   // per wave: max and min valid position
  // Q8: per key of the last four K tiles, (scale, min - 1024 scale) times
  // the score scale; slot = tile & 3
  __shared__ __attribute__((aligned(16))) float kab[Q8 ? 4 * 2 * kAT : 4];

  const int hkv = a.hkv;
  const int g = blockIdx.x % hkv;
  // Row tiles are numbered by position within each request, so a higher tile
  // of a request has more keys.  Dispatch runs largest-first: for requests
  // of equal shape, group by group from the last requests, the last row
  // tile of every request of the group, then the one before, and so on
  // (the tile numbering alone would run one request's tiles down to its
  // shortest before the next request's longest); otherwise by tile number.  When the whole grid is resident at once (two
  // workgroups per CU), the second round of slots runs smallest-first so
  // each CU pairs a long tile with a short one.
  // With key splitting, the parts of a row tile are adjacent slots.
  const int slot = static_cast<int>(blockIdx.x / hkv);
  const int rank0 = slot / a.parts;
  const int part = slot - rank0 * a.parts;
  const int rank = rank0 < a.fold_from ? rank0 : a.total_tiles - 1 - (rank0 - a.fold_from);
  int tile = a.total_tiles - 1 - rank;
  if (a.interleave > 0) {
    const int gs = a.interleave;                 // requests per group
    const int per = a.cu_tiles[1];               // row tiles of every request
    const int j = rank / (gs * per);             // group, counted from the last requests
    const int r_hi = a.b.n_req - j * gs;
    const int r_lo = max(0, r_hi - gs);
    const int lr = rank - j * gs * per;          // rank within the group
    tile = a.cu_tiles[r_lo + lr % (r_hi - r_lo)] + per - 1 - lr / (r_hi - r_lo);
  }
  const int r = find_segment(a.cu_tiles, a.b.n_req, tile);
  const int tr = tile - a.cu_tiles[r];
  const int R = a.rows_per_tile;
  const int lrow0 = tr * R;
  const int nrows = min(R, a.nrows[r] - lrow0);
  const int T = a.b.cu_T[r + 1] - a.b.cu_T[r];
  const int64_t krow0 = a.b.cu_T[r];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hf = lane >> 5;
  int pos[kQB], row_l[kQB], h[kQB];
  int64_t qrow[kQB];
  bool valid[kQB];
  const bf16_t* Q = static_cast<const bf16_t*>(a.q);
  bf16x8_t qraw[kQB][KS];
  // Every lane loads a position and a query vector, lanes past the tile's
  // rows or heads those of the tile's first row and head (their results are
  // never written): with no branch around them the loads stay in flight
  // through the position scan, which waits for the positions only.
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qv = 32 * (kQB * w + qb) + c;
    row_l[qb] = qv % R;
    const int head_l = qv / R;
    valid[qb] = head_l < a.G && row_l[qb] < nrows;
    qrow[qb] = static_cast<int64_t>(a.qrow0[r]) + lrow0 + (valid[qb] ? row_l[qb] : 0);
    h[qb] = g * a.G + (valid[qb] ? head_l : 0);
    const int p = a.q_pos ? a.q_pos[qrow[qb]] : a.pos0[r] + lrow0 + row_l[qb];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[qb][ks] = *reinterpret_cast<const bf16x8_t*>(Q + (qrow[qb] * a.hq + h[qb]) * D + ks * 16 + hf * 8);
    pos[qb] = (!valid[qb] || p < 0 || p >= T) ? -1 : p;
  }
  // Largest and smallest valid position of the tile: reduced within each
  // wave, one LDS slot per wave (atomics from every lane onto two words
  // would serialise: 4-7 us per workgroup).
  {
    int pmx = -1, pmn = 0x7fffffff;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
      if (pos[qb] >= 0) {
        pmx = max(pmx, pos[qb]);
        pmn = min(pmn, pos[qb]);
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      pmx = max(pmx, __shfl_xor(pmx, o, kWave));
      pmn = min(pmn, __shfl_xor(pmn, o, kWave));
    }
    if (lane == 0) {
      s_wpos[2 * w] = pmx;
      s_wpos[2 * w + 1] = pmn;
    }
  }
  __syncthreads();
  int pmx_all = -1, pmn_all = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < kAWaves; ++i) {
    pmx_all = max(pmx_all, s_wpos[2 * i]);
    pmn_all = min(pmn_all, s_wpos[2 * i + 1]);
  }
  // (uniform values: read once into scalar registers)
  const int klim = __builtin_amdgcn_readfirstlane(pmx_all + 1);   // keys [0, klim) are visible to someone
  const int pmin = __builtin_amdgcn_readfirstlane(pmn_all);       // keys <= pmin are visible to everyone
  const int n = klim > 0 ? ceil_div(klim, kAT) : 0;
  // leading tiles that every row sees completely need no mask
  const int n_plain = klim > 0 ? min(n, (pmin + 1) / kAT) : 0;
  // A long row tile is split into np parts of at least split_min key tiles
  // (at most a.parts); part p takes key tiles [p n / np, (p + 1) n / np) and
  // whichever part finishes last merges every part's (m, l, O) and writes.
  const int np = a.parts > 1 ? max(1, min(a.parts, n / a.split_min)) : 1;
  if (part >= np) {                               // whole workgroup: the scan is uniform
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the query loads land before the wave ends
    return;
  }
  const bool split = np > 1;
  const int t0 = part * n / np;
  const int t1 = (part + 1) * n / np;

  // MFMA operands of the queries.  bf16: the loaded vectors as they are, so
  // that nothing reads them before the first product (their loads stay in
  // flight beside the first tile copies); a lane without a valid row
  // computes on the tile's first query, is masked at every key of a masked
  // tile and is never written.  fp16 (int8-resident cache): converted, and
  // zero for lanes without a valid row.
  OpT qf[kQB][KS];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t qv = qraw[qb][ks];
      if constexpr (Q8) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          qf[qb][ks][e] = pos[qb] >= 0 ? static_cast<_Float16>(static_cast<float>(qv[e])) : static_cast<_Float16>(0.f);
      } else {
        qf[qb][ks] = qv;
      }
    }

  f32x16_t o[kQB][DB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
  float m_run[kQB], l_lane[kQB];                  // l_lane: this lane's half of the row sums
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_lane[qb] = 0.f;
  }

  const int64_t row_stride = static_cast<int64_t>(hkv) * D;
  const bf16_t* Kreq = static_cast<const bf16_t*>(a.k) + krow0 * row_stride + static_cast<int64_t>(g) * D;
  const bf16_t* Vreq = static_cast<const bf16_t*>(a.v) + krow0 * row_stride + static_cast<int64_t>(g) * D;
  // Tile copies go through buffer resources whose range ends at key klim:
  // rows past it read as zeros (those keys are masked for every row), so no
  // per-row clamp is needed.  A lane's byte offset within a tile is fixed
  // per copy instruction; the tile adds kb0 rows.
  const int rs2 = static_cast<int>(row_stride) * (Q8 ? 1 : 2);   // bytes per key row
  const u32x4_t krs = buffer_rsrc(Kreq, klim > 0 ? klim * rs2 : 0);
  const u32x4_t vrs = buffer_rsrc(Vreq, klim > 0 ? klim * rs2 : 0);
  int dvo[NDMA];
  {
    const int dma_rr = lane / CPR, dma_p = lane % CPR;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int row = (w * NDMA + j) * RPI + dma_rr;
      dvo[j] = row * rs2 + ((dma_p ^ chunk_xor<D>(row)) << 4);   // slot holds logical chunk p ^ x
    }
  }
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(kvs)) + w * NDMA * RPI * D * 2);
  auto dma_tile = [&](const u32x4_t& rs, bf16_t* dst, int kb0) __attribute__((always_inline)) {
    const int toff = kb0 * rs2;
    const uint32_t buf = static_cast<uint32_t>(dst - kvs) * 2;    // a constant at every call
#pragma unroll
    for (int j = 0; j < NDMA; ++j) buffer_copy16(rs, dvo[j] + toff, lds_w + buf + j * RPI * D * 2);
  };

  // int8-resident staging: this thread's key row of a tile and its pieces
  constexpr int NPC = D / 32;                      // 8-code pieces per thread and tensor
  const int st_row = tid >> 2;
  const int code_bytes = klim > 0 ? klim * rs2 : 0;
  const __amdgpu_buffer_rsrc_t kcr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(a.k) + krow0 * row_stride + g * D), 0, code_bytes,
      kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vcr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(a.v) + krow0 * row_stride + g * D), 0, code_bytes,
      kBufferRsrcWord3);
  const int64_t st0 = (krow0 * hkv + g) * 2;        // first stats float of this request and head
  const int st_bytes = klim > 0 ? klim * hkv * 8 : 0;
  const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(Q8 ? a.k_stats + st0 : nullptr), 0, st_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vsr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(Q8 ? a.v_stats + st0 : nullptr), 0, st_bytes, kBufferRsrcWord3);
  u32x2_t kreg[NPC], vreg[NPC];
  u32x2_t kst = {0u, 0u}, vst = {0u, 0u};
  // codes and statistics of key row kb0 + st_row (past klim: zeros)
  auto stage_load = [&](const __amdgpu_buffer_rsrc_t& cr, const __amdgpu_buffer_rsrc_t& sr, int kb0,
                        u32x2_t (&c)[NPC], u32x2_t& stv) __attribute__((always_inline)) {
    const int key = kb0 + st_row;
    const int base = key * rs2 + 8 * (tid & 3);
#pragma unroll
    for (int i = 0; i < NPC; ++i) c[i] = __builtin_amdgcn_raw_buffer_load_b64(cr, base + 32 * i, 0, 0);
    stv = __builtin_amdgcn_raw_buffer_load_b64(sr, key * hkv * 8, 0, 0);
  };
  // keys: 1024 + code as fp16 into the swizzled tile row, and the row's
  // affine map into the statistics slot of `tile`
  auto stage_commit_k = [&](const u32x2_t (&c)[NPC], const u32x2_t& stv, bf16_t* dst, int tile)
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // bytes c0..c3 -> halves 0x64 c0, 0x64 c1 and 0x64 c2, 0x64 c3
        w[2 * e] = __builtin_amdgcn_perm(0x64646464u, c[i][e], 0x04010400u);
        w[2 * e + 1] = __builtin_amdgcn_perm(0x64646464u, c[i][e], 0x04030402u);
      }
      const int piece = (tid & 3) + 4 * i;
      *reinterpret_cast<u32x4_t*>(dst + st_row * D + ((piece ^ chunk_xor<D>(st_row)) << 3)) = w;
    }
    if ((tid & 3) == 0) {
      const float mn = __uint_as_float(stv[0]), sc = __uint_as_float(stv[1]);
      float* slot = kab + (tile & 3) * (2 * kAT);
      slot[st_row] = sc * a.scale_log2;
      slot[kAT + st_row] = fmaf(-1024.f, sc, mn) * a.scale_log2;
    }
  };
  // values: min + code * scale as fp16 into the swizzled tile row, computed
  // as (1024 + code) * scale + (min - 1024 scale) from the permuted fp16
  // integer (one mixed-precision multiply-add, one rounding per value)
  auto stage_commit = [&](const u32x2_t (&c)[NPC], const u32x2_t& stv, bf16_t* dst)
      __attribute__((always_inline)) {
    const float sc = __uint_as_float(stv[1]);
    const float m2 = fmaf(-1024.f, sc, __uint_as_float(stv[0]));
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2_t x = __builtin_bit_cast(
            f16x2_t, __builtin_amdgcn_perm(0x64646464u, c[i][e >> 1], (e & 1) ? 0x04030402u : 0x04010400u));
        w[e] = pack_f16x2(fmaf(static_cast<float>(x[0]), sc, m2), fmaf(static_cast<float>(x[1]), sc, m2));
      }
      const int piece = (tid & 3) + 4 * i;
      *reinterpret_cast<u32x4_t*>(dst + st_row * D + ((piece ^ chunk_xor<D>(st_row)) << 3)) = w;
    }
  };

  // Softmax state in the log2 domain: scores enter as s * c with
  // c = sm_scale * log2(e).  The running max m_run follows the block maxima:
  // it is raised to a block's exact max whenever that exceeds it by more than
  // kRaise, so every probability is at most 2^kRaise and the key that set the
  // max has probability exactly 1 (the bf16 rounding of P then costs no more
  // than it does against the row's true max).
  constexpr float kRaise = 0.5f;
  // (Q8 scores leave key_affine already scaled)
  const float c_scale = Q8 ? 1.f : a.scale_log2;
  const f32x16_t zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bf16x2_t ones2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  const f16x2_t ones2h = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  // LDS element offsets of this lane's operand reads with the swizzle
  // resolved once (it depends on row mod 16 only).
  // K: row c of a 32-key block, channel chunk 2 ks + hf
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = c * D + (((2 * ks + hf) ^ chunk_xor<D>(c)) << 3);
  // transposed V reads: lane i of 16-lane group G reads keys 4 hf + i/4 (+8)
  // and channels 32 db + 16 (G%2) + 4 (i%4) .. +3 of a 16-key group
  const int tr_key = 4 * hf + ((lane & 15) >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int voff[2][DB];
#pragma unroll
  for (int hl = 0; hl < 2; ++hl) {
    const int row = tr_key + 8 * hl;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[hl][db] = row * D + ((((4 * db + (tr_d >> 3)) ^ chunk_xor<D>(row))) << 3) + (tr_d & 7);
  }

  // S^T for one 32-key block (keys on the MFMA rows, query vectors on lanes):
  // lane (c, hf) value i is key 8 (i/4) + 4 hf + (i%4) of the block
  auto scores = [&](const bf16_t* kt, int kb, f32x16_t (&s)[kQB]) __attribute__((always_inline)) {
    const bf16_t* kr = kt + kb * 32 * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const OpT kf = *reinterpret_cast<const OpT*>(kr + koff[ks]);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        if constexpr (Q8)
          s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[qb][ks], ks == 0 ? zero16 : s[qb], 0, 0, 0);
        else
          s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ks], ks == 0 ? zero16 : s[qb], 0, 0, 0);
      }
    }
  };
  // Q8: channel sum of each query vector (both lane halves)
  float sumq[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    float sq = 0.f;
    if constexpr (Q8) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) sq += static_cast<float>(qf[qb][ks][e]);
      sq += __shfl_xor(sq, 32, kWave);
    }
    sumq[qb] = sq;
  }
  // Q8: scores of block kb0 from q . (1024 + c) to log2-domain logits,
  // s * A_key + B_key * sum(q); before the mask (a constant key row has A = 0)
  auto key_affine = [&](f32x16_t (&s)[kQB], int kb0) __attribute__((always_inline)) {
    const float* ab = kab + ((kb0 >> 6) & 3) * (2 * kAT) + (kb0 & 32) + 4 * hf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t A = *reinterpret_cast<const f32x4_t*>(ab + 8 * j);
      const f32x4_t B = *reinterpret_cast<const f32x4_t*>(ab + kAT + 8 * j);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[qb][4 * j + e] = fmaf(A[e], s[qb][4 * j + e], B[e] * sumq[qb]);
    }
  };
  // masked keys -> -inf (keys past a row's position; kb0 = block's first key)
  auto apply_mask = [&](f32x16_t (&s)[kQB], int kb0) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int lim = pos[qb] - kb0 - 4 * hf;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) > lim) s[qb][i] = -INFINITY;
    }
  };
  // probabilities as bf16 pairs against the running max; the row sum is
  // taken over exactly the bf16 values the V product consumes.  Returns this
  // block's lane-local sums.
  auto probs = [&](const f32x16_t (&s)[kQB], uint32_t (&pk)[kQB][8], float (&lb)[kQB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float neg_m = m_run[qb] == -INFINITY ? 0.f : -m_run[qb];
      lb[qb] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][2 * i], c_scale, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][2 * i + 1], c_scale, neg_m));
        if constexpr (Q8) {
          pk[qb][i] = pack_f16x2(p0, p1);
          lb[qb] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk[qb][i]), ones2h, lb[qb], false);
        } else {
          pk[qb][i] = pack_bf16x2(p0, p1);
          lb[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[qb][i]), ones2, lb[qb], false);
        }
      }
    }
  };
  // Max of one block's scores in the log2 domain, over both lane halves
  // (v_permlane32_swap exchanges the halves without going through LDS).
  auto block_max = [&](const f32x16_t (&s)[kQB], float (&bm)[kQB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float m = fmaxf(s[qb][0], s[qb][1]);
#pragma unroll
      for (int i = 2; i < 16; ++i) m = fmaxf(m, s[qb][i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      bm[qb] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c_scale;
    }
  };
  // Set the running max from block s, given as the first block (exact).
  auto init_max = [&](const f32x16_t (&s)[kQB]) __attribute__((always_inline)) {
    float bm[kQB];
    block_max(s, bm);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) m_run[qb] = bm[qb];
  };
  // O is kept against the max its latest V product used; alpha_pend takes it
  // to the max of the block whose V product comes next.
  float alpha_pend[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) alpha_pend[qb] = 1.f;
  auto catch_up = [&]() __attribute__((always_inline)) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) any = any || alpha_pend[qb] != 1.f;
    if (__any(any)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha_pend[qb];
        alpha_pend[qb] = 1.f;
      }
    }
  };
  // O^T += V^T P^T for one 32-key block of tile vt
  auto pv = [&](const bf16_t* vt, int kb, const uint32_t (&pk)[kQB][8]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      OpT pb[kQB];
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const u32x4_t pw = {pk[qb][4 * st], pk[qb][4 * st + 1], pk[qb][4 * st + 2], pk[qb][4 * st + 3]};
        pb[qb] = __builtin_bit_cast(OpT, pw);
      }
      const bf16_t* vblk = vt + (kb * 32 + 16 * st) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vblk + voff[0][db]));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vblk + voff[1][db]));
        const s16x4_t vv[2] = {lo, hi};
        const OpT vf = __builtin_bit_cast(OpT, vv);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          if constexpr (Q8)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pb[qb], o[qb][db], 0, 0, 0);
          else
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[qb], o[qb][db], 0, 0, 0);
        }
      }
    }
  };

  // Software pipeline over 32-key blocks b: one half step runs the score
  // MFMAs of block b+1, the softmax of block b and the V product of block
  // b-1 in one branch-free stretch (the V product lags by a block so that
  // its MFMAs never wait for this block's exponentials).  Per tile t there is
  // one barrier (B), after which K_{t+2} and V_{t+1} are copied into the
  // buffers of K_t and V_{t-1}: the half step before B still reads those,
  // the one after B reads K_{t+1} and V_t, which the barrier waited for.
  f32x16_t s_a[kQB], s_b[kQB];                     // scores of blocks 0 and 1 of a tile
  uint32_t pk_a[kQB][8], pk_b[kQB][8];             // probabilities of blocks 0 and 1
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int i = 0; i < 8; ++i) pk_b[qb][i] = 0u;  // "block -1": contributes nothing
  // sc: scores of block b (first key kb0); kt/kbs: K tile and block of b+1
  // into sn; vt/kbp/pkp: V tile, block and probabilities of b-1; pkc gets b's.
  // The rescale of O for block b's max is applied before the V product of
  // block b (in the next half step), after that of block b-1.
  auto half_step = [&](f32x16_t (&sc)[kQB], int kb0, bool masked, const bf16_t* kt, int kbs,
                       f32x16_t (&sn)[kQB], const bf16_t* vt, int kbp, const uint32_t (&pkp)[kQB][8],
                       uint32_t (&pkc)[kQB][8]) __attribute__((always_inline)) {
    if constexpr (Q8) key_affine(sc, kb0);
    if (masked) apply_mask(sc, kb0);
    catch_up();
    // From here one branch-free stretch: the score MFMAs of b+1 and the V
    // MFMAs of b-1 beside the softmax of b, so the scheduler can interleave
    // them (the raise of the running max is a select, not a branch).
    scores(kt, kbs, sn);
    pv(vt, kbp, pkp);
    float bm[kQB], lb[kQB];
    block_max(sc, bm);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const bool up = bm[qb] > m_run[qb] + kRaise;
      const float al = __builtin_amdgcn_exp2f(m_run[qb] - bm[qb]);   // m_run = -inf: 0 (O, l are 0)
      alpha_pend[qb] = up ? al : 1.f;
      l_lane[qb] *= alpha_pend[qb];
      m_run[qb] = up ? bm[qb] : m_run[qb];
    }
    probs(sc, pkc, lb);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) l_lane[qb] += lb[qb];
    // Keep this block's softmax in this half step: without these uses the
    // compiler sinks it past the barrier into the next half step, which then
    // holds two blocks' softmax while this one holds only MFMAs.
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pkc[qb][i]));
      asm volatile("" ::"v"(l_lane[qb]), "v"(m_run[qb]), "v"(alpha_pend[qb]));
    }
  };
  // tile t: kc holds K_t, kn K_{t+1}; vc holds V_t, vp V_{t-1}
  auto tile_step = [&](int t, bf16_t* kc, const bf16_t* kn, const bf16_t* vc, bf16_t* vp)
      __attribute__((always_inline)) {
    const bool masked = t >= n_plain;
    // S(2t+1) from K_t, softmax(2t), P(2t-1) V_{t-1}
    half_step(s_a, t * kAT, masked, kc, 1, s_b, vp, 1, pk_b, pk_a);
    // B: K_{t+1} and V_t landed everywhere; K_t and V_{t-1} free
    if constexpr (Q8) {
      // this wave's tile writes done (its register loads are awaited by the
      // compiler where the commits below use them)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (t + 2 < t1) stage_commit_k(kreg, kst, kc, t + 2);
      if (t + 1 < t1) stage_commit(vreg, vst, vp);
      if (t + 3 < t1) stage_load(kcr, ksr, (t + 3) * kAT, kreg, kst);
      if (t + 2 < t1) stage_load(vcr, vsr, (t + 2) * kAT, vreg, vst);
    } else {
      copies_landed_barrier<0>();
      if (t + 2 < t1) dma_tile(krs, kc, (t + 2) * kAT);
      if (t + 1 < t1) dma_tile(vrs, vp, (t + 1) * kAT);
    }
    // S(2t+2) from K_{t+1} (unused after the last tile), softmax(2t+1), P(2t) V_t
    half_step(s_b, t * kAT + 32, masked, kn, 0, s_a, vc, 0, pk_a, pk_b);
  };

  if (t1 > t0) {
    if constexpr (Q8) {
      stage_load(kcr, ksr, t0 * kAT, kreg, kst);
      stage_load(vcr, vsr, t0 * kAT, vreg, vst);
      stage_commit_k(kreg, kst, k0s, t0);
      stage_commit(vreg, vst, v0s);
      if (t0 + 1 < t1) {
        stage_load(kcr, ksr, (t0 + 1) * kAT, kreg, kst);
        stage_commit_k(kreg, kst, k1s, t0 + 1);
      }
      // the first tile step commits K_{t0+2} and V_{t0+1}
      if (t0 + 2 < t1) stage_load(kcr, ksr, (t0 + 2) * kAT, kreg, kst);
      if (t0 + 1 < t1) stage_load(vcr, vsr, (t0 + 1) * kAT, vreg, vst);
    } else {
      dma_tile(krs, k0s, t0 * kAT);
      dma_tile(vrs, v0s, t0 * kAT);
      if (t0 + 1 < t1) dma_tile(krs, k1s, (t0 + 1) * kAT);
    }
    // the first half step multiplies zero probabilities with "V_{t0-1}"
    for (int i = tid; i < TILE / 8; i += kAThreads)
      *reinterpret_cast<u32x4_t*>(v1s + 8 * i) = u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (Q8)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      copies_landed_barrier<0>();
    scores(k0s, 0, s_a);
    if constexpr (Q8) {
      // the first half step maps s_a itself; the max is taken from a copy
      f32x16_t s0[kQB];
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) s0[qb] = s_a[qb];
      key_affine(s0, t0 * kAT);
      if (t0 >= n_plain) apply_mask(s0, t0 * kAT);
      init_max(s0);                                 // the first block sets the max exactly
    } else {
      if (t0 >= n_plain) apply_mask(s_a, t0 * kAT);
      init_max(s_a);                                // the first block sets the max exactly
    }
  }
  // Every global load the compiler tracks (Q) has completed here on all
  // paths; saying so keeps it from waiting for them, and so for the tile
  // copies behind them, inside the loop (vmcnt(0), expcnt and lgkmcnt free).
  if constexpr (!Q8) __builtin_amdgcn_s_waitcnt(0x0F70);
  // two tiles per trip so every buffer is a distinct static array
  int tl = t0;                                      // last tile processed
  for (int t = t0; t < t1; t += 2) {
    tile_step(t, k0s, k1s, v0s, v1s);
    tl = t;
    if (t + 1 >= t1) break;
    tile_step(t + 1, k1s, k0s, v1s, v0s);
    tl = t + 1;
  }
  // P(last block) V_{last tile}
  if (t1 > t0) {
    catch_up();
    if (((tl - t0) & 1) == 0) pv(v0s, 1, pk_b);
    else pv(v1s, 1, pk_b);
  }

  if (split) {
    // Partial state of this part in 16-byte chunks, chunk-major so that a
    // wave's store of one chunk is 1 KB contiguous: per query block the
    // unnormalised O (DB x 4 chunks), then (m, the lane's half of l, 0, 0).
    // The chunks are stored and loaded with device-scope coherence, which
    // reaches across the XCDs' L2 caches; every wave waits for its stores to
    // be acknowledged before the barrier that precedes the counter bump
    // (stores_done_barrier), so the last arrival reads complete partials.
    constexpr int NC = kQB * (DB * 4 + 1);
    const int64_t item = static_cast<int64_t>(tile) * hkv + g;
    const __amdgpu_buffer_rsrc_t pr = handoff_rsrc(
        a.ws_part, static_cast<int64_t>(a.total_tiles) * hkv * a.parts * NC * kAThreads * 16);
    // lane part of a chunk's offset, and its uniform part (a scalar offset)
    const uint32_t lane_off = static_cast<uint32_t>(tid) * 16;
    auto chunk_off = [&](int pt, int c) __attribute__((always_inline)) {
      return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
          static_cast<int>(((item * a.parts + pt) * NC + c) * kAThreads * 16)));
    };
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const f32x4_t v = {o[qb][db][4 * c4], o[qb][db][4 * c4 + 1], o[qb][db][4 * c4 + 2],
                             o[qb][db][4 * c4 + 3]};
          put_dev4(pr, lane_off, chunk_off(part, qb * (DB * 4 + 1) + db * 4 + c4), v);
        }
      const f32x4_t ml = {m_run[qb], l_lane[qb], 0.f, 0.f};
      put_dev4(pr, lane_off, chunk_off(part, qb * (DB * 4 + 1) + DB * 4), ml);
    }
    stores_done_barrier();                        // every wave's stores have completed
    if (tid == 0)
      s_pos[0] = __hip_atomic_fetch_add(&a.ws_cnt[item], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_pos[0] != np - 1) return;               // not the last to finish: it merges
    for (int op = 0; op < np; ++op) {
      if (op == part) continue;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const f32x4_t ml = get_dev4(pr, lane_off, chunk_off(op, qb * (DB * 4 + 1) + DB * 4));
        const float m2 = ml[0], l2 = ml[1];
        const float mm = fmaxf(m_run[qb], m2);
        const float mu = mm == -INFINITY ? 0.f : mm;
        const float a1 = __builtin_amdgcn_exp2f(m_run[qb] - mu), a2 = __builtin_amdgcn_exp2f(m2 - mu);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const f32x4_t v = get_dev4(pr, lane_off, chunk_off(op, qb * (DB * 4 + 1) + db * 4 + c4));
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) o[qb][db][4 * c4 + e4] = o[qb][db][4 * c4 + e4] * a1 + v[e4] * a2;
          }
        l_lane[qb] = l_lane[qb] * a1 + l2 * a2;
        m_run[qb] = mm;
      }
    }
    // every part has arrived: leave the counter zero for the next call
    if (tid == 0) __hip_atomic_store(&a.ws_cnt[item], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    if (!valid[qb] || pos[qb] < 0) continue;
    const float l = l_lane[qb] + __shfl_xor(l_lane[qb], 32, kWave);
    const int64_t orow = static_cast<int64_t>(a.orow0[r]) + lrow0 + row_l[qb];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16_t* O = static_cast<bf16_t*>(a.out) + (orow * a.hq + h[qb]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * hf;
        u32x2_t pk2;
        pk2[0] = pack_bf16x2(o[qb][db][4 * i] * inv, o[qb][db][4 * i + 1] * inv);
        pk2[1] = pack_bf16x2(o[qb][db][4 * i + 2] * inv, o[qb][db][4 * i + 3] * inv);
        *reinterpret_cast<u32x2_t*>(O + d0) = pk2;
      }
    if (a.lse && hf == 0) a.lse[orow * a.hq + h[qb]] = (m_run[qb] + log2f(l)) * kLn2;
  }
}

template <int D, bool Q8>
static hipError_t launch_attn_mfma(const AttnArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_mfma_kernel<D, Q8>), grid, dim3(kAThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 kernel: one wave per (row, head)
// ---------------------------------------------------------------------------
constexpr int kFT = 128;         // key granularity of the fp32 statistics splits

template <bool STATS_ONLY>
__global__ void __launch_bounds__(256) attn_f32_kernel(AttnArgs a, int d, int total_rows) {
  const int wid = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & 63;
  if (wid >= total_rows * a.hq) return;
  const int orow_g = wid / a.hq, h = wid % a.hq;
  // locate the request of this output row
  int r = 0;
  while (r + 1 < a.b.n_req && a.orow0[r + 1] <= orow_g) ++r;
  const int i = orow_g - a.orow0[r];
  if (i >= a.nrows[r]) return;
  const int64_t qrow = static_cast<int64_t>(a.qrow0[r]) + i;
  const int T = a.b.cu_T[r + 1] - a.b.cu_T[r];
  int pos = a.q_pos ? a.q_pos[qrow] : a.pos0[r] + i;
  if (pos < 0 || pos >= T) return;
  const int g = h / a.G;
  const int64_t krow0 = a.b.cu_T[r];
  const float* Q = static_cast<const float*>(a.q) + (qrow * a.hq + h) * d;
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);
  int kbeg = 0, klim = pos + 1;
  if constexpr (STATS_ONLY) {
    kbeg = blockIdx.y * a.split_keys;
    klim = min(klim, kbeg + a.split_keys);
  }
  float m_run = -INFINITY, l_run = 0.f;
  float o0 = 0.f, o1 = 0.f;                       // channels lane, lane + 64
  for (int kb0 = kbeg; kb0 < klim; kb0 += 64) {
    const int key = kb0 + lane;
    float s = -INFINITY;
    if (key < klim) {
      const float* kr = K + ((krow0 + key) * a.hkv + g) * d;
      float acc = 0.f;
      for (int e = 0; e < d; ++e) acc = fmaf(Q[e], kr[e], acc);
      s = acc * a.scale_log2;
    }
    const float mx = wave_max(s);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    const float p = exp2f(s - m_use);
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
    if constexpr (!STATS_ONLY) {
      o0 *= alpha;
      o1 *= alpha;
      const int nk = min(64, klim - kb0);
      for (int jj = 0; jj < nk; ++jj) {
        const float pj = __shfl(p, jj, kWave);
        const float* vr = V + ((krow0 + kb0 + jj) * a.hkv + g) * d;
        o0 = fmaf(pj, vr[lane], o0);
        if (d > 64) o1 = fmaf(pj, vr[lane + 64], o1);
      }
    }
  }
  const int64_t orow = orow_g;
  if constexpr (STATS_ONLY) {
    if (lane == 0) {
      const int64_t idx = static_cast<int64_t>(blockIdx.y) * a.plane + orow * a.hq + h;
      a.part_m[idx] = m_run;
      a.part_l[idx] = l_run;
    }
  } else {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* O = static_cast<float*>(a.out) + (orow * a.hq + h) * d;
    O[lane] = o0 * inv;
    if (d > 64) O[lane + 64] = o1 * inv;
    if (a.lse && lane == 0) a.lse[orow * a.hq + h] = (m_run + log2f(l_run)) * kLn2;
  }
}

static void fill_tiles(AttnArgs& a, int R) {
  a.rows_per_tile = R;
  a.cu_tiles[0] = 0;
  for (int r = 0; r < a.b.n_req; ++r) a.cu_tiles[r + 1] = a.cu_tiles[r] + ceil_div(a.nrows[r], R);
  a.total_tiles = a.cu_tiles[a.b.n_req];
}

static int rows_per_tile(int G) { return G >= kAQ ? 1 : kAQ / G; }

// Key splitting: only grids that one dispatch round holds (two workgroups
// per CU) have too few workgroups to even out tiles of unequal length, so
// only they get the workspace.  The part count fills one dispatch round: two
// parts when the row tiles nearly fill it, up to kSplitMaxParts for the few
// row tiles of a small recompute set (a handful of seam windows, say).  A
// row tile is cut into parts of at least kSplitMinTiles key tiles, or
// kSplitMinTilesSmall when the grid is that small.
constexpr int kSplitMaxItems = 2 * kCUs;
constexpr int kSplitMinTiles = 12;
constexpr int kSplitMinTilesSmall = 6;
constexpr int kSplitMaxParts = 8;

// Workspace: arrival counters first, at a fixed offset and size, so that
// calls of any shape can share one zero-filled workspace (every completed
// call leaves the counters zero); the parts' partial results after them.
constexpr size_t kAttnCntBytes = 4096;
static_assert(kSplitMaxItems * sizeof(int) <= kAttnCntBytes, "counter region");

struct AttnSplitLayout {
  int64_t items = 0;             // row tiles x kv heads
  int parts = 1;
  size_t off_part = 0, bytes = 0;
};

static AttnSplitLayout attn_split_layout(const kvf_layer_desc& L, const BatchArgs& B,
                                         const int32_t* cu_q) {
  AttnSplitLayout s;
  if (L.dtype != KVF_BF16) return s;
  const int R = rows_per_tile(L.n_q_heads / L.n_kv_heads);
  int64_t tiles = 0;
  for (int r = 0; r < B.n_req; ++r) tiles += ceil_div(cu_q[r + 1] - cu_q[r], R);
  const int64_t items = tiles * L.n_kv_heads;
  if (items == 0 || items > kSplitMaxItems) return s;
  const int64_t chunks = kQB * (L.head_dim / 32 * 4 + 1);   // 16-byte chunks per thread and part
  s.items = items;
  s.parts = static_cast<int>(std::min<int64_t>(
      kSplitMaxParts, std::max<int64_t>(2, (kSplitMaxItems + items - 1) / items)));
  s.off_part = kAttnCntBytes;
  s.bytes = s.off_part + static_cast<size_t>(items * s.parts * chunks * kAThreads) * 16;
  return s;
}

size_t attention_workspace(const kvf_layer_desc& L, const BatchArgs& B, const int32_t* cu_q) {
  return attn_split_layout(L, B, cu_q).bytes;
}

// kst/vst non-null: fk/fv are the 8-bit codes of an int8-resident cache
static hipError_t attention_impl(const kvf_layer_desc& L, const BatchArgs& B, const void* q,
                                 const int32_t* q_pos, const int32_t* cu_q, const void* fk,
                                 const void* fv, const float* kst, const float* vst, float sm_scale,
                                 void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t st) {
  const bool q8 = kst != nullptr;
  AttnArgs a{};
  a.b = B;
  for (int r = 0; r < B.n_req; ++r) {
    a.qrow0[r] = cu_q[r];
    a.orow0[r] = cu_q[r];
    a.nrows[r] = cu_q[r + 1] - cu_q[r];
    a.pos0[r] = 0;
  }
  a.q = q;
  a.q_pos = q_pos;
  a.k = fk;
  a.v = fv;
  a.k_stats = kst;
  a.v_stats = vst;
  a.out = out;
  a.lse = lse;
  a.hq = L.n_q_heads;
  a.hkv = L.n_kv_heads;
  a.G = L.n_q_heads / L.n_kv_heads;
  a.scale_log2 = sm_scale * kLog2e;
  a.n_splits = 1;
  a.parts = 1;
  if (L.dtype == KVF_BF16) {
    fill_tiles(a, rows_per_tile(a.G));
    const int64_t tiles = static_cast<int64_t>(a.total_tiles) * a.hkv;
    if (tiles == 0) return hipSuccess;
    const AttnSplitLayout sl = attn_split_layout(L, B, cu_q);
    if (sl.bytes > 0 && ws != nullptr && ws_bytes >= sl.bytes) {
      a.parts = sl.parts;
      a.split_min = sl.parts > 2 ? kSplitMinTilesSmall : kSplitMinTiles;
      a.ws_cnt = static_cast<int*>(ws);
      a.ws_part = reinterpret_cast<float*>(static_cast<char*>(ws) + sl.off_part);
    }
    const int64_t blocks = tiles * a.parts;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    // without splitting, a grid that one dispatch round holds runs its second
    // round smallest-first, pairing long and short tiles on a CU
    a.fold_from = a.parts == 1 && blocks <= 2 * kCUs ? std::max(1, kCUs / a.hkv) : a.total_tiles;
    // Several requests with the same row tiles and length: interleave them
    // longest-first, so the long row tiles of the last requests do not start
    // late and end the kernel alone (Qwen2.5-3B-shaped batch, 16 requests x
    // 33 row tiles x 2 kv heads: attention 181 -> 152 us).  A grid of at most
    // four dispatch rounds interleaves the whole batch; larger grids
    // interleave pairs of requests, so the workgroups in flight share the
    // keys and values of two requests in the caches instead of all of them
    // (Qwen3-8B-shaped batch, 8 x 100 row tiles x 8 kv heads, 12.5 rounds:
    // the whole batch interleaved was 3% slower than request order).
    a.interleave = 0;
    if (B.n_req > 1) {
      bool same = true;
      const int per = a.cu_tiles[1], T0 = B.cu_T[1] - B.cu_T[0];
      for (int r = 1; r < B.n_req && same; ++r)
        same = a.cu_tiles[r + 1] - a.cu_tiles[r] == per && B.cu_T[r + 1] - B.cu_T[r] == T0;
      a.interleave = same && per > 0 ? (blocks <= 4 * 2 * kCUs ? B.n_req : 2) : 0;
    }
    hipError_t e;
    if (q8)
      e = L.head_dim == 128 ? launch_attn_mfma<128, true>(a, dim3(blocks), st)
                            : launch_attn_mfma<64, true>(a, dim3(blocks), st);
    else
      e = L.head_dim == 128 ? launch_attn_mfma<128, false>(a, dim3(blocks), st)
                            : launch_attn_mfma<64, false>(a, dim3(blocks), st);
    if (e != hipSuccess) return e;
  } else {
    if (q8) return hipErrorInvalidValue;
    const int total_rows = cu_q[B.n_req];
    const int64_t waves = static_cast<int64_t>(total_rows) * a.hq;
    hipLaunchKernelGGL((attn_f32_kernel<false>), dim3(ceil_div(static_cast<int>(waves), 4)),
                       dim3(256), 0, st, a, L.head_dim, total_rows);
  }
  return hipGetLastError();
}

hipError_t launch_attention(const kvf_layer_desc& L, const BatchArgs& B, const void* q,
                            const int32_t* q_pos, const int32_t* cu_q, const void* fk,
                            const void* fv, float sm_scale, void* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  return attention_impl(L, B, q, q_pos, cu_q, fk, fv, nullptr, nullptr, sm_scale, out, lse, ws,
                        ws_bytes, st);
}

hipError_t launch_attention_q8(const kvf_layer_desc& L, const BatchArgs& B, const void* q,
                               const int32_t* q_pos, const int32_t* cu_q, const kvf_q8_cache& c,
                               float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                               hipStream_t st) {
  return attention_impl(L, B, q, q_pos, cu_q, c.k_codes, c.v_codes, c.k_stats, c.v_stats,
                        sm_scale, out, lse, ws, ws_bytes, st);
}

// ---------------------------------------------------------------------------
// attention mass
// ---------------------------------------------------------------------------
// Three launches for bf16:
//  1. mass_stats_bf16_kernel: per (128-key chunk, kv head), the softmax
//     statistics (max, sum) of every used query vector over the chunk's
//     visible keys.  S^T = K Q^T with the chunk's keys held in registers as
//     the MFMA A operand and query vectors staged in LDS as B, so each lane
//     owns one query vector's scores.
//  2. lse_combine_kernel: chunk statistics -> log2-domain LSE per (row, head).
//  3. mass_colsum_bf16_kernel: per (128-key tile, kv head), S = Q K^T again
//     (query vectors on the MFMA rows, keys on the lanes), exp(s - lse)
//     summed over the query vectors of the group; the last kv head of a key
//     tile to finish adds the heads in a fixed order (deterministic).
// The "last to finish" hand-off counts arrivals in the workspace, which must
// be zero before the first call; each call leaves the counters zero.
// fp32: statistics by the fp32 attention kernel, column sums by one wave per
// (key, kv head).

// Combine split statistics into log2-domain LSE per (row, head).
// Large planes: a block takes E = 64 consecutive entries and 256 / E groups of
// splits (group k takes every (256 / E)-th split from k); lane = entry, so
// each load reads 256 contiguous bytes of one statistics plane.  The groups'
// (max, sum) pairs are combined in a fixed order.
template <int E>
__global__ void __launch_bounds__(256) lse_combine_kernel(const float* __restrict__ pm,
                                                          const float* __restrict__ pl, int n_splits,
                                                          int64_t plane, int64_t n,
                                                          float* __restrict__ lse2) {
  constexpr int NG = 256 / E;
  __shared__ float s_m[NG][E], s_l[NG][E];
  const int e = threadIdx.x % E, grp = threadIdx.x / E;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * E + e;
  float m = -INFINITY, l = 0.f;
  auto add = [&](float ms, float ls) {
    if (ms > m) {
      l = l * (m == -INFINITY ? 0.f : exp2f(m - ms)) + ls;
      m = ms;
    } else if (ms > -INFINITY) {
      l += ls * exp2f(ms - m);
    }
  };
  if (i < n) {
    for (int sp = grp; sp < n_splits; sp += 4 * NG) {   // four loads of each plane in flight
      float ms[4], ls[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = sp + NG * u < n_splits;
        ms[u] = ok ? pm[(sp + NG * u) * plane + i] : -INFINITY;
        ls[u] = ok ? pl[(sp + NG * u) * plane + i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) add(ms[u], ls[u]);
    }
  }
  s_m[grp][e] = m;
  s_l[grp][e] = l;
  __syncthreads();
  if (grp == 0 && i < n) {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) add(s_m[k][e], s_l[k][e]);
    lse2[i] = l > 0.f ? m + log2f(l) : INFINITY;   // INFINITY: contributes nothing
  }
}

// Small planes (too few entries to fill the chip 64 at a time): one wave per
// entry, lanes over splits.
__global__ void __launch_bounds__(256) lse_combine_wave_kernel(const float* __restrict__ pm,
                                                               const float* __restrict__ pl, int n_splits,
                                                               int64_t plane, int64_t n,
                                                               float* __restrict__ lse2) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (i >= n) return;
  float m = -INFINITY, l = 0.f;
  for (int sp = lane; sp < n_splits; sp += kWave) {
    const float ms = pm[sp * plane + i], ls = pl[sp * plane + i];
    if (ms > m) {
      l = l * (m == -INFINITY ? 0.f : exp2f(m - ms)) + ls;
      m = ms;
    } else if (ms > -INFINITY) {
      l += ls * exp2f(ms - m);
    }
  }
  const float mw = wave_max(m);
  const float lw = wave_sum(m > -INFINITY ? l * exp2f(m - mw) : 0.f);
  if (lane == 0) lse2[i] = lw > 0.f ? mw + log2f(lw) : INFINITY;   // INFINITY: contributes nothing
}

struct MassArgs {
  BatchArgs b;
  int qrow0[KVF_MAX_REQ];        // first q_u row used by each request
  int nq[KVF_MAX_REQ];           // query rows used
  int pos0[KVF_MAX_REQ];         // position of the first used query row
  int orow0[KVF_MAX_REQ];        // their rows in lse2 / the statistics planes
  int cu_ktiles[KVF_MAX_REQ + 1];
  int total_ktiles;
  const void* q;
  const void* k;
  const float* lse2;             // [rows, Hq]
  float* part;                   // [Hkv, sum N]
  float* part_m;                 // [chunks, rows, Hq] (statistics pass)
  float* part_l;
  int64_t plane;                 // rows * Hq
  int hq, hkv, G;
  float scale_log2;
  // Arrival counters (zero between calls): the last column-sum workgroup of
  // a key tile adds the kv heads.
  int* cnt_cols;                 // [total_ktiles]
  ScoreOut out;                  // scores [sum N]
  // keys-only re-positioning fused into the statistics pass (ROT): the
  // chunk table, per-chunk keys and rope tables of kvf_rerotate; k_rw is the
  // fused K cache the pass writes the re-positioned keys to
  const kvf_chunk* rot_chunks;
  int rot_n;
  const bf16_t* pool_k;
  int64_t pool_rows;
  const float* rope_cos;
  const float* rope_sin;
  int rope_n;
  bf16_t* k_rw;
};

constexpr int kMK = 128;         // keys per workgroup (4 waves x 32)
// Query vectors staged per round (LDS), MQS: 256 when a request has at most
// that many (one round), else 128, whose smaller LDS and register footprint
// lets three workgroups share a CU instead of two, so one's products overlap
// another's exponentials (measured 6% faster with 2048 vectors, 3% slower
// with 256).
constexpr int kMQSOne = 256;
constexpr int kMQSMany = 128;

// ROT: the pass also re-positions the context keys (kvf_rerotate, keys
// only): a key row that a chunk covers is read from the per-chunk cache
// (pool row src_row + t), turned by R(pos0) of that chunk, scored, and
// written to its fused row by the first query part (blockIdx.z == 0), so the
// column-sum pass and everything after read the fused cache as kvf_rerotate
// leaves it; rows no chunk covers (the query rows) are read from the fused
// cache as they are.  With the per-chunk cache in the fused cache itself (in
// place), the launch must not split the query vectors (gridDim.z == 1): a
// second part could read a key the first has already turned.
template <int D, int kMQS, bool ROT>
__global__ void __launch_bounds__(256) mass_stats_bf16_kernel(MassArgs a) {
  constexpr int KS = D / 16;
  constexpr int LDQ = D + 8;     // padded rows: B-fragment reads hit distinct banks
  constexpr int VPR = D / 8;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[kMQS][LDQ];
  __shared__ float2 st[4][kMQS];
  const int hkv = a.hkv;
  const int g = blockIdx.x % hkv;
  const int chunk = static_cast<int>(blockIdx.x / hkv);
  const int r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hf = lane >> 5;
  const int T = a.b.cu_T[r + 1] - a.b.cu_T[r];
  const int64_t krow0 = a.b.cu_T[r];
  const int nqv = a.nq[r] * a.G;
  // blockIdx.z splits the query vectors into gridDim.z parts (multiples of
  // 32) so that small grids put more workgroups on the chip
  const int per = ceil_div(ceil_div(nqv, static_cast<int>(gridDim.z)), 32) * 32;
  const int q_lo = min(nqv, static_cast<int>(blockIdx.z) * per);
  const int q_hi = min(nqv, q_lo + per);
  const int key0 = chunk * kMK;
  const int64_t out0 = static_cast<int64_t>(chunk) * a.plane;
  if (key0 >= T) {          // past this request's keys: an empty chunk
    for (int qv = q_lo + tid; qv < q_hi; qv += 256) {
      const int row = qv / a.G, hl = qv - row * a.G;
      const int64_t idx = out0 + (static_cast<int64_t>(a.orow0[r]) + row) * a.hq + g * a.G + hl;
      a.part_m[idx] = -INFINITY;
      a.part_l[idx] = 0.f;
    }
    return;
  }
  // every key of the chunk is visible to every used query vector (their
  // positions are pos0, pos0 + 1, ..): no mask
  const bool full = key0 + kMK <= min(a.pos0[r] + 1, T);
  // this wave's 32 keys as the A operand: row = key, k = 8 hf + e
  const bf16_t* Kg = static_cast<const bf16_t*>(a.k);
  const int key_a = key0 + 32 * w + c;
  int kp = -1;                                    // ROT: the key's chunk start position
  const bf16_t* krow = Kg + ((krow0 + key_a) * hkv + g) * D + hf * 8;
  if constexpr (ROT) {
    // the chunk covering this lane's key row: the wave's lanes test 64
    // chunks at a time against the wave's 32 rows, and the few that
    // intersect are broadcast to every lane
    const int64_t row = krow0 + key_a;
    const int64_t w_lo = krow0 + key0 + 32 * w;
    const int64_t w_hi = min(w_lo + 32, krow0 + T);
    int ksrc = 0;
    for (int base = 0; base < a.rot_n; base += kWave) {
      const int ci = base + lane;
      kvf_chunk chn{};
      bool hit = false;
      if (ci < a.rot_n) {
        chn = a.rot_chunks[ci];
        hit = chn.len > 0 && chn.src_row >= 0 && static_cast<int64_t>(chn.src_row) + chn.len <= a.pool_rows &&
              chn.pos0 >= 0 && chn.pos0 < a.rope_n && chn.dst_row < w_hi &&
              static_cast<int64_t>(chn.dst_row) + chn.len > w_lo;
      }
      for (uint64_t hits = __ballot(hit); hits != 0; hits &= hits - 1) {
        const int l = __builtin_ctzll(hits);
        const int dst = __shfl(chn.dst_row, l, kWave), len = __shfl(chn.len, l, kWave);
        const int p0 = __shfl(chn.pos0, l, kWave), src = __shfl(chn.src_row, l, kWave);
        if (key_a < T && row >= dst && row < static_cast<int64_t>(dst) + len) {
          kp = p0;
          ksrc = src + static_cast<int>(row - dst);
        }
      }
    }
    if (kp >= 0) krow = a.pool_k + (static_cast<int64_t>(ksrc) * hkv + g) * D + hf * 8;
  }
  bf16x8_t kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (key_a < T) {
      kf[ks] = *reinterpret_cast<const bf16x8_t*>(krow + ks * 16);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[ks][e] = static_cast<__bf16>(0.f);
    }
  }
  // ROT: re-position this lane's key (when a chunk covers it) and write it
  // to the fused cache (first query part only); this lane holds channels
  // 16 ks + 8 hf + e, and the partner of channel j < D/2 is j + D/2, in
  // k-step ks + KS/2 of the same lane
  auto rotate_keys = [&]() __attribute__((always_inline)) {
    if (kp < 0) return;
    const float* cr = a.rope_cos + static_cast<int64_t>(kp) * (D / 2) + hf * 8;
    const float* sr = a.rope_sin + static_cast<int64_t>(kp) * (D / 2) + hf * 8;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      float cv[8], sv[8];
      Elem<float>::load8(cr + ks * 16, cv);
      Elem<float>::load8(sr + ks * 16, sv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = static_cast<float>(kf[ks][e]), y = static_cast<float>(kf[ks + KS / 2][e]);
        kf[ks][e] = static_cast<__bf16>(fmaf(x, cv[e], -(y * sv[e])));
        kf[ks + KS / 2][e] = static_cast<__bf16>(fmaf(y, cv[e], x * sv[e]));
      }
    }
    if (blockIdx.z == 0) {
      bf16_t* Kw = a.k_rw + ((krow0 + key_a) * hkv + g) * D + hf * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<bf16x8_t*>(Kw + ks * 16) = kf[ks];
    }
  };
  const bf16_t* Qg = static_cast<const bf16_t*>(a.q);
  const float cs = a.scale_log2;
  for (int qs = q_lo; qs < q_hi; qs += kMQS) {
    const int qe = min(q_hi, qs + kMQS);
    // stage this round's query vectors (zero rows past the end): all loads
    // in flight together, then the stores
    constexpr int NV = kMQS * VPR / 256;
    u32x4_t v4[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = tid + 256 * j;
      const int qq = idx / VPR, vc = idx - qq * VPR;
      const int qi = qs + qq;
      v4[j] = u32x4_t{0u, 0u, 0u, 0u};
      if (qi < qe) {
        const int row = qi / a.G, hl = qi - row * a.G;
        v4[j] = *reinterpret_cast<const u32x4_t*>(
            Qg + ((static_cast<int64_t>(a.qrow0[r]) + row) * a.hq + g * a.G + hl) * D + vc * 8);
      }
    }
    if (qs == 0) {          // the K fragments have been in flight alongside
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(kf[ks]));
    }
    if (ROT && qs == q_lo) rotate_keys();   // while this round's query loads are in flight
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = tid + 256 * j;
      const int qq = idx / VPR, vc = idx - qq * VPR;
      *reinterpret_cast<u32x4_t*>(&Qs[qq][vc * 8]) = v4[j];
    }
    __syncthreads();
    // four independent 32-vector blocks at a time (four MFMA chains in flight)
#pragma unroll 1
    for (int b0 = 0; b0 < qe - qs; b0 += 128) {
      f32x16_t s[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[j][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8_t qfrag = *reinterpret_cast<const bf16x8_t*>(&Qs[b0 + 32 * j + c][ks * 16 + hf * 8]);
          s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qfrag, s[j], 0, 0, 0);
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // lane c: query vector qs + b0 + 32 j + c; keys key0 + 32 w + 8 (i/4) + 4 hf + (i%4)
        const int qv = qs + b0 + 32 * j + c;
        // raw scores: the max commutes with the positive scale, which goes
        // into the exponent's multiply-add
        float sv[16];
        if (full) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[i] = s[j][i];
        } else {
          const int pos = a.pos0[r] + qv / a.G;
          const int lim = min(pos, T - 1) - (key0 + 32 * w + 4 * hf);
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[i] = 8 * (i >> 2) + (i & 3) <= lim ? s[j][i] : -INFINITY;
        }
        float m = sv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, sv[i]);
        m = fmaxf(m, __shfl_xor(m, 32, kWave)) * cs;
        float l = 0.f;
        if (m > -INFINITY) {
#pragma unroll
          for (int i = 0; i < 16; ++i) l += __builtin_amdgcn_exp2f(fmaf(sv[i], cs, -m));
        }
        l += __shfl_xor(l, 32, kWave);
        if (hf == 0) st[w][b0 + 32 * j + c] = make_float2(m, l);
      }
    }
    __syncthreads();
    for (int qv = qs + tid; qv < qe; qv += 256) {
      float m = -INFINITY, l = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float2 x = st[ww][qv - qs];
        if (x.x > m) {
          l = l * (m == -INFINITY ? 0.f : exp2f(m - x.x)) + x.y;
          m = x.x;
        } else if (x.x > -INFINITY) {
          l += x.y * exp2f(x.x - m);
        }
      }
      const int row = qv / a.G, hl = qv - row * a.G;
      const int64_t idx = out0 + (static_cast<int64_t>(a.orow0[r]) + row) * a.hq + g * a.G + hl;
      a.part_m[idx] = m;
      a.part_l[idx] = l;
    }
    __syncthreads();
  }
  if (ROT && q_lo >= q_hi) rotate_keys();   // no query vectors here: the keys still move
}

constexpr int kMQB = 128;        // query vectors staged per column-sum round

template <int D>
__global__ void __launch_bounds__(256) mass_colsum_bf16_kernel(MassArgs a) {
  constexpr int KS = D / 16;
  constexpr int LDQ = D + 8;
  constexpr int VPR = D / 8;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[kMQB][LDQ];
  __shared__ float Ls[kMQB];
  const int g = blockIdx.x % a.hkv;
  const int kt = static_cast<int>(blockIdx.x / a.hkv);
  const int r = find_segment(a.cu_ktiles, a.b.n_req, kt);
  const int key0 = (kt - a.cu_ktiles[r]) * kMK;
  const int N = a.b.n_ctx[r];
  const int64_t krow0 = a.b.cu_T[r];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hf = lane >> 5;
  const int key = key0 + 32 * w + c;
  const bool kvalid = key < N;

  // K fragments (B operand of S = Q K^T): key = lane column
  const bf16_t* Kg = static_cast<const bf16_t*>(a.k);
  bf16x8_t kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (kvalid) {
      kf[ks] = *reinterpret_cast<const bf16x8_t*>(Kg + ((krow0 + key) * a.hkv + g) * D + ks * 16 + hf * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[ks][e] = static_cast<__bf16>(0.f);
    }
  }
  const bf16_t* Qg = static_cast<const bf16_t*>(a.q);
  // blockIdx.y splits the query vectors into gridDim.y parts (multiples of
  // 32), each summed by its own workgroup; the last arrival of a key tile
  // adds every (part, kv head) sum
  const int nqv_all = a.nq[r] * a.G;
  const int per = ceil_div(ceil_div(nqv_all, static_cast<int>(gridDim.y)), 32) * 32;
  const int q_lo = min(nqv_all, static_cast<int>(blockIdx.y) * per);
  const int nqv = min(nqv_all, q_lo + per);
  float colsum = 0.f;
  for (int q0 = q_lo; q0 < nqv; q0 += kMQB) {
    // this round's query vectors and LSEs: all loads in flight together
    constexpr int NV = kMQB * VPR / 256;
    u32x4_t v4[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = tid + 256 * j;
      const int qq = idx / VPR, vc = idx - qq * VPR;
      const int qi = q0 + qq;
      v4[j] = u32x4_t{0u, 0u, 0u, 0u};
      if (qi < nqv) {
        const int row = qi / a.G, hl = qi - row * a.G;
        v4[j] = *reinterpret_cast<const u32x4_t*>(
            Qg + ((static_cast<int64_t>(a.qrow0[r]) + row) * a.hq + g * a.G + hl) * D + vc * 8);
      }
    }
    float l2 = INFINITY;
    if (tid < kMQB) {
      const int qi = q0 + tid;
      if (qi < nqv) {
        const int row = qi / a.G, hl = qi - row * a.G;
        l2 = a.lse2[(static_cast<int64_t>(a.orow0[r]) + row) * a.hq + g * a.G + hl];
      }
    }
    if (q0 == 0) {          // the K fragments have been in flight alongside
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(kf[ks]));
    }
    __syncthreads();        // previous round's reads of Qs and Ls are done
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = tid + 256 * j;
      const int qq = idx / VPR, vc = idx - qq * VPR;
      *reinterpret_cast<u32x4_t*>(&Qs[qq][vc * 8]) = v4[j];
    }
    if (tid < kMQB) Ls[tid] = l2;
    __syncthreads();
    // the four 32-vector blocks as four independent MFMA chains
    f32x16_t s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[j][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t qfrag = *reinterpret_cast<const bf16x8_t*>(&Qs[32 * j + c][ks * 16 + hf * 8]);
        s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfrag, kf[ks], s[j], 0, 0, 0);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qq = 32 * j + 8 * (i >> 2) + 4 * hf + (i & 3);
        colsum += __builtin_amdgcn_exp2f(s[j][i] * a.scale_log2 - Ls[qq]);   // Ls = +inf: padding -> 0
      }
  }
  colsum += __shfl_xor(colsum, 32, kWave);
  const int n_all = a.b.cu_N[a.b.n_req];
  // column sums [query part][kv head][sum N], moved as plain buffer accesses
  // with the device-scope cache policy so a batch of them is in flight at
  // once (relaxed atomics would go one at a time)
  const int n_sum = a.hkv * static_cast<int>(gridDim.y);    // partial sums per key
  const __amdgpu_buffer_rsrc_t pr = handoff_rsrc(a.part, static_cast<int64_t>(n_sum) * n_all * 4);
  if (hf == 0 && kvalid)
    put_dev1(pr, static_cast<uint32_t>(a.b.cu_N[r] + key) * 4,
             static_cast<uint32_t>(blockIdx.y * a.hkv + g) * n_all * 4, colsum);
  // the last arrival of this key tile adds the partial sums in a fixed order
  __shared__ int s_flag;
  if (!arrive_last(a.cnt_cols + kt, n_sum, &s_flag)) return;
  if (tid < kMK && key0 + tid < N) {
    const uint32_t key_off = static_cast<uint32_t>(a.b.cu_N[r] + key0 + tid) * 4;
    float sum = 0.f;
    for (int g0 = 0; g0 < n_sum; g0 += 8) {
      float pv8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        pv8[u] = get_dev1(pr, key_off, static_cast<uint32_t>(min(g0 + u, n_sum - 1)) * n_all * 4);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (g0 + u < n_sum) sum += pv8[u];
    }
    store_score(a.out, a.b.cu_N[r] + key0 + tid, sum);
  }
}

// fp32: one wave per (context key, kv head)
__global__ void __launch_bounds__(256) mass_colsum_f32_kernel(MassArgs a, int d) {
  const int wid = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & 63;
  const int total = a.b.cu_N[a.b.n_req];
  if (wid >= total * a.hkv) return;
  const int g = wid % a.hkv, t = wid / a.hkv;
  const int r = find_segment(a.b.cu_N, a.b.n_req, t);
  const int key = t - a.b.cu_N[r];
  const float* kr = static_cast<const float*>(a.k) + ((static_cast<int64_t>(a.b.cu_T[r]) + key) * a.hkv + g) * d;
  const float* Qg = static_cast<const float*>(a.q);
  const int nqv = a.nq[r] * a.G;
  float acc = 0.f;
  for (int qi = lane; qi < nqv; qi += 64) {
    const int row = qi / a.G, hl = qi - row * a.G;
    const float* qr = Qg + ((static_cast<int64_t>(a.qrow0[r]) + row) * a.hq + g * a.G + hl) * d;
    float dot = 0.f;
    for (int e = 0; e < d; ++e) dot = fmaf(qr[e], kr[e], dot);
    const float l2 = a.lse2[(static_cast<int64_t>(a.orow0[r]) + row) * a.hq + g * a.G + hl];
    acc += exp2f(dot * a.scale_log2 - l2);
  }
  acc = wave_sum(acc);
  if (lane == 0) a.part[static_cast<int64_t>(g) * total + t] = acc;
}

__global__ void __launch_bounds__(256) head_sum_kernel(const float* __restrict__ part, int hkv,
                                                       int n, ScoreOut out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int g = 0; g < hkv; ++g) s += part[static_cast<int64_t>(g) * n + i];
  store_score(out, i, s);
}

// Arrival counters of the attention-mass workspace: one per 128-key tile of
// context, at workspace offset 0 in a region of fixed size.
constexpr size_t kMassCntBytes = 65536;
constexpr int64_t kMassMaxKeyTiles = kMassCntBytes / sizeof(int);

int64_t attn_mass_key_tiles(const BatchArgs& B) {
  int64_t ktiles = 0;
  for (int r = 0; r < B.n_req; ++r) ktiles += ceil_div(B.n_ctx[r], kMK);
  return ktiles;
}

// Query-vector parts of a small grid's statistics and column-sum passes.
constexpr int kMassQParts = 2;

namespace {
struct MassLayout {
  int64_t rows;          // query rows used (sum over requests)
  int n_splits;
  int split_keys;
  size_t off_pm, off_pl, off_lse, off_part, off_cnt, total;
  int64_t n_cnt;         // arrival counters: one per key tile
};

MassLayout mass_layout(const kvf_layer_desc& L, const BatchArgs& B, int n_last_q) {
  MassLayout m{};
  int max_T = 0;
  for (int r = 0; r < B.n_req; ++r) {
    const int U = B.cu_T[r + 1] - B.cu_T[r] - B.n_ctx[r];
    const int nq = n_last_q > 0 ? std::min(n_last_q, U) : U;
    m.rows += nq;
    max_T = std::max(max_T, B.cu_T[r + 1] - B.cu_T[r]);
  }
  if (L.dtype == KVF_BF16) {
    // statistics per 128-key chunk
    m.split_keys = kMK;
    m.n_splits = std::max(1, ceil_div(max_T, kMK));
  } else {
    // fp32 statistics kernel: enough splits to cover the chip twice
    const int64_t base = std::max<int64_t>(1, m.rows * L.n_q_heads / 4);
    const int key_tiles = std::max(1, ceil_div(max_T, kFT));
    int splits = static_cast<int>(std::min<int64_t>(key_tiles, ceil_div(512, static_cast<int>(std::min<int64_t>(base, 512)))));
    splits = std::max(1, std::min(splits, 64));
    m.split_keys = ceil_div(key_tiles, splits) * kFT;
    m.n_splits = ceil_div(std::max(max_T, 1), m.split_keys);
  }
  const int64_t plane = m.rows * L.n_q_heads;
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  int64_t ktiles = 0;
  for (int r = 0; r < B.n_req; ++r) ktiles += ceil_div(B.n_ctx[r], kMK);
  m.n_cnt = ktiles;
  // arrival counters first, at a fixed offset and size: calls of any shape
  // can share one zero-filled workspace
  m.off_cnt = 0;
  m.off_pm = kMassCntBytes;
  m.off_pl = align(m.off_pm + sizeof(float) * plane * m.n_splits);
  m.off_lse = align(m.off_pl + sizeof(float) * plane * m.n_splits);
  m.off_part = align(m.off_lse + sizeof(float) * plane);
  // column sums of up to kMassQParts query parts per kv head and key
  m.total = align(m.off_part + sizeof(float) * kMassQParts * static_cast<size_t>(L.n_kv_heads) * B.cu_N[B.n_req]);
  return m;
}
}  // namespace

size_t attn_mass_workspace(const kvf_layer_desc& L, const BatchArgs& B, int n_last_q) {
  return mass_layout(L, B, n_last_q).total;
}

hipError_t launch_attn_mass(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                            const void* q_u, int n_last_q, const ScoreOut& out, void* ws,
                            size_t ws_bytes, hipStream_t st, const MassRotate* rot) {
  const MassLayout lay = mass_layout(L, B, n_last_q);
  if (ws_bytes < lay.total || lay.n_cnt > kMassMaxKeyTiles) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  float* pm = reinterpret_cast<float*>(base + lay.off_pm);
  float* pl = reinterpret_cast<float*>(base + lay.off_pl);
  float* lse2 = reinterpret_cast<float*>(base + lay.off_lse);
  float* part = reinterpret_cast<float*>(base + lay.off_part);
  int* cnt = reinterpret_cast<int*>(base + lay.off_cnt);
  const int G = L.n_q_heads / L.n_kv_heads;
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(L.head_dim));
  const int64_t plane = lay.rows * L.n_q_heads;
  if (plane > 0x7fffffff) return hipErrorInvalidValue;

  MassArgs m{};
  m.b = B;
  int orow = 0;
  for (int r = 0; r < B.n_req; ++r) {
    const int U = B.cu_T[r + 1] - B.cu_T[r] - B.n_ctx[r];
    const int nq = n_last_q > 0 ? std::min(n_last_q, U) : U;
    m.qrow0[r] = B.cu_U[r] + (U - nq);
    m.nq[r] = nq;
    m.pos0[r] = B.n_ctx[r] + (U - nq);
    m.orow0[r] = orow;
    orow += nq;
    m.cu_ktiles[r + 1] = m.cu_ktiles[r] + ceil_div(B.n_ctx[r], kMK);
  }
  m.total_ktiles = m.cu_ktiles[B.n_req];
  m.q = q_u;
  m.k = fk;
  m.lse2 = lse2;
  m.part = part;
  m.part_m = pm;
  m.part_l = pl;
  m.plane = plane;
  m.hq = L.n_q_heads;
  m.hkv = L.n_kv_heads;
  m.G = G;
  m.scale_log2 = scale_log2;
  m.cnt_cols = cnt;
  m.out = out;
  // the re-positioning rides on the bf16 statistics pass; without one (no
  // query rows, or fp32) it runs as its own keys-only kvf_rerotate launch
  const bool fused_rot = rot != nullptr && L.dtype == KVF_BF16 && plane > 0;
  if (rot != nullptr && !fused_rot) {
    const hipError_t e = launch_rerotate(L, rot->chunks, rot->n_chunks, rot->max_len, rot->pool_k,
                                         nullptr, nullptr, rot->pool_rows, rot->rope_cos,
                                         rot->rope_sin, rot->rope_n, const_cast<void*>(fk), nullptr,
                                         rot->fused_rows, 1, st);
    if (e != hipSuccess) return e;
  }
  if (fused_rot) {
    m.rot_chunks = rot->chunks;
    m.rot_n = rot->n_chunks;
    m.pool_k = static_cast<const bf16_t*>(rot->pool_k);
    m.pool_rows = rot->pool_rows;
    m.rope_cos = rot->rope_cos;
    m.rope_sin = rot->rope_sin;
    m.rope_n = rot->rope_n;
    m.k_rw = static_cast<bf16_t*>(const_cast<void*>(fk));
  }
  const int n = B.cu_N[B.n_req];
  if (plane == 0) {
    // no query rows: every key gets zero mass
    if (n > 0) {
      hipLaunchKernelGGL(head_sum_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st, part, 0, n,
                         out);
    }
    return hipGetLastError();
  }

  // pass 1: softmax statistics of the used query rows
  if (L.dtype == KVF_BF16) {
    int nqv_max = 0;
    for (int r = 0; r < B.n_req; ++r) nqv_max = std::max(nqv_max, m.nq[r] * m.G);
    // a grid under two workgroups per CU with at least 256 query vectors per
    // request splits them in two (128-vector rounds, three workgroups per CU)
    const int64_t wgs = static_cast<int64_t>(lay.n_splits) * m.hkv * B.n_req;
    // (not when re-positioning in place: a second part could read a key the
    // first has already turned)
    const bool in_place = fused_rot && rot->pool_k == fk;
    const int nqp = (!in_place && wgs < 2 * kCUs && nqv_max >= kMassQParts * kMQSMany) ? kMassQParts : 1;
    const dim3 grid(lay.n_splits * m.hkv, B.n_req, nqp);
    const int per = ceil_div(ceil_div(nqv_max, nqp), 32) * 32;
    const bool one = per > kMQSMany && per <= kMQSOne;
#define KVF_MASS_STATS(D_, Q_)                                                                   \
  do {                                                                                           \
    if (fused_rot) hipLaunchKernelGGL((mass_stats_bf16_kernel<D_, Q_, true>), grid, dim3(256), 0, st, m); \
    else hipLaunchKernelGGL((mass_stats_bf16_kernel<D_, Q_, false>), grid, dim3(256), 0, st, m); \
  } while (0)
    if (L.head_dim == 128) {
      if (one) KVF_MASS_STATS(128, kMQSOne);
      else KVF_MASS_STATS(128, kMQSMany);
    } else {
      if (one) KVF_MASS_STATS(64, kMQSOne);
      else KVF_MASS_STATS(64, kMQSMany);
    }
#undef KVF_MASS_STATS
  } else {
    AttnArgs a{};
    a.b = B;
    for (int r = 0; r < B.n_req; ++r) {
      a.qrow0[r] = m.qrow0[r];
      a.nrows[r] = m.nq[r];
      a.pos0[r] = m.pos0[r];
      a.orow0[r] = m.orow0[r];
    }
    a.plane = plane;
    a.q = q_u;
    a.q_pos = nullptr;
    a.k = fk;
    a.part_m = pm;
    a.part_l = pl;
    a.n_splits = lay.n_splits;
    a.split_keys = lay.split_keys;
    a.hq = L.n_q_heads;
    a.hkv = L.n_kv_heads;
    a.G = G;
    a.scale_log2 = scale_log2;
    const dim3 grid(ceil_div(static_cast<int>(plane), 4), lay.n_splits);
    hipLaunchKernelGGL((attn_f32_kernel<true>), grid, dim3(256), 0, st, a, L.head_dim,
                       static_cast<int>(lay.rows));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (plane >= 64 * kCUs)
    hipLaunchKernelGGL(lse_combine_kernel<64>, dim3(ceil_div(static_cast<int>(plane), 64)), dim3(256), 0, st,
                       pm, pl, lay.n_splits, plane, plane, lse2);
  else
    hipLaunchKernelGGL(lse_combine_wave_kernel, dim3(ceil_div(static_cast<int>(plane), 256 / kWave)),
                       dim3(256), 0, st, pm, pl, lay.n_splits, plane, plane, lse2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // pass 2: normalised probabilities summed per context key and kv head
  if (n == 0) return hipSuccess;
  if (L.dtype == KVF_BF16) {
    const int64_t blocks = static_cast<int64_t>(m.total_ktiles) * m.hkv;
    // a grid under two workgroups per CU whose requests have more than one
    // round of query vectors splits them over kMassQParts workgroups
    int nqv_max = 0;
    for (int r = 0; r < B.n_req; ++r) nqv_max = std::max(nqv_max, m.nq[r] * m.G);
    const int nqp = (blocks < 2 * kCUs && nqv_max > kMQB) ? kMassQParts : 1;
    const dim3 grid(static_cast<unsigned>(blocks), nqp);
    if (L.head_dim == 128)
      hipLaunchKernelGGL(mass_colsum_bf16_kernel<128>, grid, dim3(256), 0, st, m);
    else
      hipLaunchKernelGGL(mass_colsum_bf16_kernel<64>, grid, dim3(256), 0, st, m);
  } else {
    const int64_t waves = static_cast<int64_t>(n) * m.hkv;
    hipLaunchKernelGGL(mass_colsum_f32_kernel, dim3(ceil_div(static_cast<int>(waves), 4)),
                       dim3(256), 0, st, m, L.head_dim);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // (bf16: the column-sum pass added the heads)
  if (L.dtype != KVF_BF16)
    hipLaunchKernelGGL(head_sum_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st, part, L.n_kv_heads,
                       n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// attention mass without a caller workspace
// ---------------------------------------------------------------------------
// For callers that cannot allocate device memory: the workspace lives in this
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes the array's name (a host-side stand-in) to a
// kernel: its device address is looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[KVF_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

hipError_t mass_scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_attn_mass_noalloc(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                                    const void* q_u, int n_last_q, const ScoreOut& out,
                                    hipStream_t st) {
  const MassLayout lay = mass_layout(L, B, n_last_q);
  if (lay.total > KVF_NOALLOC_SCRATCH_BYTES) return hipErrorInvalidValue;
  void* ws = nullptr;
  hipError_t e = mass_scratch_address(&ws);
  if (e != hipSuccess) return e;
  // the arrival counters this call uses start at zero whatever an earlier
  // call left (a fill kernel, which graph capture records safely)
  if (lay.n_cnt > 0) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>(ceil_div(static_cast<int>(lay.n_cnt), 256))),
                       dim3(256), 0, st, reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + lay.off_cnt),
                       lay.n_cnt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_attn_mass(L, B, fk, q_u, n_last_q, out, ws, KVF_NOALLOC_SCRATCH_BYTES, st);
}

}  // namespace kvf
