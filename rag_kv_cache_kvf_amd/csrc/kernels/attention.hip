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
// fp32 path: one wave per (row, head) with lane-parallel keys; used by the
// small fp32 workloads only.
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
  int rows_per_tile;             // R
  const void* q;
  const int32_t* q_pos;
  const void* k;
  const void* v;
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
// 8 waves: wave w owns query vectors [32*(w%4), +32) and key half w/4 of every
// 128-key tile.  K and V tiles are copied global -> LDS by the DMA path
// (global_load_lds, 16 bytes per lane, no registers involved) into two
// static buffers: tile t+1 streams in while tile t is computed.  Both tiles
// are row-major with the 16-byte chunks of row r XOR-swizzled (chunk_xor), so
// the key-row reads of the score MFMA and the transposing reads of V
// (ds_read_b64_tr_b16, one 4-key x 4-channel transpose per 16 lanes) hit
// distinct banks.
constexpr int kAT = 128;         // keys per tile (two halves of 64)
constexpr int kAThreads = 512;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_cvoid_t;

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

template <int D>
__global__ void __launch_bounds__(kAThreads) attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 16;       // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;       // 32-channel output blocks
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;    // rows per DMA instruction (64 lanes x 16 B)
  constexpr int NDMA = kAT / RPI / 8;   // DMA instructions per wave per tile and tensor
  constexpr int TILE = kAT * D;
  __shared__ __attribute__((aligned(16))) bf16_t k0s[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t k1s[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t v0s[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t v1s[TILE];
  __shared__ int s_pos[2];

  const int hkv = a.hkv;
  const int g = blockIdx.x % hkv;
  const int tile = a.total_tiles - 1 - static_cast<int>(blockIdx.x / hkv);
  const int r = find_segment(a.cu_tiles, a.b.n_req, tile);
  const int tr = tile - a.cu_tiles[r];
  const int R = a.rows_per_tile;
  const int lrow0 = tr * R;
  const int nrows = min(R, a.nrows[r] - lrow0);
  const int T = a.b.cu_T[r + 1] - a.b.cu_T[r];
  const int64_t krow0 = a.b.cu_T[r];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qg = w & 3, kg = w >> 2;
  const int c = lane & 31, hf = lane >> 5;
  const int qv = 32 * qg + c;
  const int row_l = qv % R, head_l = qv / R;
  const bool valid = head_l < a.G && row_l < nrows;
  const int64_t qrow = static_cast<int64_t>(a.qrow0[r]) + lrow0 + row_l;
  const int h = g * a.G + head_l;
  int pos = -1;
  if (valid) {
    pos = a.q_pos ? a.q_pos[qrow] : a.pos0[r] + lrow0 + row_l;
    if (pos < 0 || pos >= T) pos = -1;
  }
  if (tid == 0) {
    s_pos[0] = -1;                 // max position
    s_pos[1] = 0x7fffffff;         // min position
  }
  __syncthreads();
  if (pos >= 0) {
    atomicMax(&s_pos[0], pos);
    atomicMin(&s_pos[1], pos);
  }
  __syncthreads();
  const int kend = s_pos[0] + 1;                  // keys [0, kend) are visible to someone
  const int pmin = s_pos[1];                      // keys <= pmin are visible to everyone

  const int kbeg = 0, klim = kend;

  const bf16_t* Q = static_cast<const bf16_t*>(a.q);
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (pos >= 0) {
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(Q + (qrow * a.hq + h) * D + ks * 16 + hf * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = static_cast<__bf16>(0.f);
    }
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // per-request base of this kv head; rows are row_stride elements apart
  const int64_t row_stride = static_cast<int64_t>(hkv) * D;
  const bf16_t* Kreq = static_cast<const bf16_t*>(a.k) + krow0 * row_stride + static_cast<int64_t>(g) * D;
  const bf16_t* Vreq = static_cast<const bf16_t*>(a.v) + krow0 * row_stride + static_cast<int64_t>(g) * D;
  // this lane's DMA slot: row lane / CPR of each group, physical chunk lane % CPR
  const int dma_rr = lane / CPR, dma_p = lane % CPR;

  auto dma_tile = [&](const bf16_t* src_req, bf16_t* dst, int kb0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int grp = w * NDMA + j;
      const int row = grp * RPI + dma_rr;
      const int q = dma_p ^ chunk_xor<D>(row);            // logical chunk held by this slot
      const int key = min(kb0 + row, klim - 1);           // tail rows repeat a valid key
      const bf16_t* src = src_req + static_cast<int64_t>(key) * row_stride + q * 8;
      __builtin_amdgcn_global_load_lds((global_cvoid_t*)(src), (lds_void_t*)(dst + grp * RPI * D), 16, 0, 0);
    }
  };

  // Softmax state in the log2 domain: scores enter as s * c with
  // c = sm_scale * log2(e).  The running max m_run is raised only when a
  // tile's max exceeds it by more than kSlack (then O and l are rescaled);
  // otherwise probabilities are taken against the old max and may exceed 1
  // by at most 2^kSlack, which fp32 sums and bf16 operands carry exactly as
  // well.  The result is the same softmax, with far fewer rescales.
  constexpr float kSlack = 8.f;
  const float c_scale = a.scale_log2;
  const f32x16_t zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bf16x2_t ones2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  // LDS element offsets of this lane's operand reads, with the XOR swizzle
  // resolved once: the swizzle term depends only on row mod 16, which the
  // 32-key and 16-key block steps (multiples of 16 rows) do not change.
  // K rows 64 kg + 32 kb + c, channel chunk 2 kk + hf:
  int koff[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    koff[kk] = (64 * kg + c) * D + (((2 * kk + hf) ^ chunk_xor<D>(c)) << 3);
  // transposed V reads: lane i of 16-lane group G reads keys 4 hf + i/4 (+8)
  // and channels 32 db + 16 (G%2) + 4 (i%4) .. +3
  const int tr_key = 4 * hf + ((lane & 15) >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int voff[2][DB];
#pragma unroll
  for (int hl = 0; hl < 2; ++hl) {
    const int row = tr_key + 8 * hl;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[hl][db] = (64 * kg + row) * D + ((((4 * db + (tr_d >> 3)) ^ chunk_xor<D>(row))) << 3) + (tr_d & 7);
  }

  // One 128-key tile computed from (ks, vs).  MASK selects the variant that
  // applies the causal and range mask (only the last tiles need it).
  auto step = [&](const bf16_t* ks_, const bf16_t* vs_, int kb0, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k_half = kb0 + 64 * kg;             // first key of this wave's half
    if (k_half >= klim) return;                   // wave-uniform
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16_t* krow = ks_ + kb * 32 * D;      // + koff: row 64 kg + 32 kb + c
      const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(krow + koff[0]);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[0], zero16, 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < KS; ++kk) {
        const bf16x8_t kfrag = *reinterpret_cast<const bf16x8_t*>(krow + koff[kk]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[kk], s[kb], 0, 0, 0);
      }
    }
    if constexpr (MASK) {
      // key = k_half + 32 kb + 8 (i/4) + 4 hf + (i%4) is visible iff key <= lim
      const int lim = min(pos, klim - 1) - k_half - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 2 : 0); i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c_scale;     // tile max, log2 domain
    if (__builtin_expect(__any(mx > m_run + kSlack), 0)) {
      asm volatile("; rescale");                  // keeps this rare path a branch
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    float rs = 0.f;
    {
      uint32_t pk[2][8];                          // bf16 probability pairs
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * i], c_scale, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * i + 1], c_scale, neg_m));
          pk[kb][i] = pack_bf16x2(p0, p1);
          // normalise by the sum of the bf16 values the V product consumes
          rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[kb][i]), ones2, rs, false);
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4_t pw = {pk[kb][4 * st], pk[kb][4 * st + 1], pk[kb][4 * st + 2], pk[kb][4 * st + 3]};
          const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
          const bf16_t* vblk = vs_ + (kb * 32 + 16 * st) * D;   // + voff: this lane's rows
          // keep each 16-key group's V reads next to its MFMAs (register pressure)
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vblk + voff[0][db]));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vblk + voff[1][db]));
            const s16x4_t vv[2] = {lo, hi};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pb,
                                                            o[db], 0, 0, 0);
          }
        }
      }
    }
    rs += __shfl_xor(rs, 32, kWave);
    l_run += rs;
  };

  const int ntiles = klim > kbeg ? ceil_div(klim - kbeg, kAT) : 0;
  // leading tiles every row sees completely need no mask
  int n_plain = 0;
  if (pmin >= kbeg) n_plain = min(min(ntiles, (pmin + 1 - kbeg) / kAT), (klim - kbeg) / kAT);
  auto run_tile = [&](int t, const bf16_t* ks_, const bf16_t* vs_) __attribute__((always_inline)) {
    if (t < n_plain)
      step(ks_, vs_, kbeg + t * kAT, std::false_type{});
    else
      step(ks_, vs_, kbeg + t * kAT, std::true_type{});
  };
  if (ntiles > 0) {
    dma_tile(Kreq, k0s, kbeg);
    dma_tile(Vreq, v0s, kbeg);
  }
  __syncthreads();                                // waits for the DMA (vmcnt) too
  // two tiles per trip so every buffer is a distinct static array
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 1 < ntiles) {
      dma_tile(Kreq, k1s, kbeg + (t + 1) * kAT);
      dma_tile(Vreq, v1s, kbeg + (t + 1) * kAT);
    }
    run_tile(t, k0s, v0s);
    __syncthreads();
    if (t + 1 >= ntiles) break;
    if (t + 2 < ntiles) {
      dma_tile(Kreq, k0s, kbeg + (t + 2) * kAT);
      dma_tile(Vreq, v0s, kbeg + (t + 2) * kAT);
    }
    run_tile(t + 1, k1s, v1s);
    __syncthreads();
  }

  // merge the two key halves: waves 4..7 hand (m, l, O) to waves 0..3
  const int slot = qg * 64 + lane;
  float* xo0 = reinterpret_cast<float*>(k0s);     // O blocks [0, DB/2)
  float* xo1 = reinterpret_cast<float*>(k1s);     // O blocks [DB/2, DB)
  float* xml = reinterpret_cast<float*>(v0s);
  constexpr int HO = 8 * DB;                      // floats per lane in each O half
  if (kg == 1) {
    xml[2 * slot] = m_run;
    xml[2 * slot + 1] = l_run;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float* dstp = db < DB / 2 ? xo0 : xo1;
        dstp[slot * HO + (db % (DB / 2)) * 16 + i] = o[db][i];
      }
  }
  __syncthreads();
  if (kg == 1) return;
  {
    const float m2 = xml[2 * slot];
    const float l2 = xml[2 * slot + 1];
    const float mm = fmaxf(m_run, m2);
    const float mu = mm == -INFINITY ? 0.f : mm;
    const float a1 = __builtin_amdgcn_exp2f(m_run - mu), a2 = __builtin_amdgcn_exp2f(m2 - mu);
    l_run = l_run * a1 + l2 * a2;
    m_run = mm;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* srcp = db < DB / 2 ? xo0 : xo1;
        o[db][i] = o[db][i] * a1 + srcp[slot * HO + (db % (DB / 2)) * 16 + i] * a2;
      }
  }

  if (!valid || pos < 0) return;
  const int64_t orow = static_cast<int64_t>(a.orow0[r]) + lrow0 + row_l;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  bf16_t* O = static_cast<bf16_t*>(a.out) + (orow * a.hq + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = db * 32 + 8 * i + 4 * hf;
      u32x2_t pk2;
      pk2[0] = pack_bf16x2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv);
      pk2[1] = pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
      *reinterpret_cast<u32x2_t*>(O + d0) = pk2;
    }
  if (a.lse && hf == 0) a.lse[orow * a.hq + h] = (m_run + log2f(l_run)) * kLn2;
}

template <int D>
static hipError_t launch_attn_bf16(const AttnArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_bf16_kernel<D>), grid, dim3(kAThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 kernel: one wave per (row, head)
// ---------------------------------------------------------------------------
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

hipError_t launch_attention(const kvf_layer_desc& L, const BatchArgs& B, const void* q,
                            const int32_t* q_pos, const int32_t* cu_q, const void* fk,
                            const void* fv, float sm_scale, void* out, float* lse,
                            hipStream_t st) {
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
  a.out = out;
  a.lse = lse;
  a.hq = L.n_q_heads;
  a.hkv = L.n_kv_heads;
  a.G = L.n_q_heads / L.n_kv_heads;
  a.scale_log2 = sm_scale * kLog2e;
  a.n_splits = 1;
  if (L.dtype == KVF_BF16) {
    fill_tiles(a, rows_per_tile(a.G));
    const int64_t blocks = static_cast<int64_t>(a.total_tiles) * a.hkv;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const hipError_t e = L.head_dim == 128 ? launch_attn_bf16<128>(a, dim3(blocks), st)
                                           : launch_attn_bf16<64>(a, dim3(blocks), st);
    if (e != hipSuccess) return e;
  } else {
    const int total_rows = cu_q[B.n_req];
    const int64_t waves = static_cast<int64_t>(total_rows) * a.hq;
    hipLaunchKernelGGL((attn_f32_kernel<false>), dim3(ceil_div(static_cast<int>(waves), 4)),
                       dim3(256), 0, st, a, L.head_dim, total_rows);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// attention mass
// ---------------------------------------------------------------------------
// Three launches (bf16):
//  1. mass_stats_bf16_kernel: per (128-key chunk, kv head), the softmax
//     statistics (max, sum) of every used query vector over the chunk's
//     visible keys.  S^T = K Q^T with the chunk's keys held in registers as
//     the MFMA A operand and query vectors staged in LDS as B, so each lane
//     owns one query vector's scores.
//  2. lse_combine_kernel: chunk statistics -> log2-domain LSE per (row, head).
//  3. mass_colsum_bf16_kernel: per (128-key tile, kv head), S = Q K^T again
//     (query vectors on the MFMA rows, keys on the lanes), exp(s - lse)
//     summed over the query vectors of the group.
//  4. head_sum_kernel: the kv heads added in a fixed order (deterministic).
// fp32: statistics by the fp32 attention kernel, column sums by one wave per
// (key, kv head).

// combine split statistics into log2-domain LSE per (row, head): one wave per
// entry, lanes over splits
__global__ void __launch_bounds__(256) lse_combine_kernel(const float* __restrict__ pm,
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
};

constexpr int kMK = 128;         // keys per workgroup (4 waves x 32)
constexpr int kMQS = 256;        // query vectors staged per round (LDS)

template <int D>
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
  const int key0 = chunk * kMK;
  const int64_t out0 = static_cast<int64_t>(chunk) * a.plane;
  if (key0 >= T) {          // past this request's keys: an empty chunk
    for (int qv = tid; qv < nqv; qv += 256) {
      const int row = qv / a.G, hl = qv - row * a.G;
      const int64_t idx = out0 + (static_cast<int64_t>(a.orow0[r]) + row) * a.hq + g * a.G + hl;
      a.part_m[idx] = -INFINITY;
      a.part_l[idx] = 0.f;
    }
    return;
  }
  // this wave's 32 keys as the A operand: row = key, k = 8 hf + e
  const bf16_t* Kg = static_cast<const bf16_t*>(a.k);
  const int key_a = key0 + 32 * w + c;
  bf16x8_t kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (key_a < T) {
      kf[ks] = *reinterpret_cast<const bf16x8_t*>(Kg + ((krow0 + key_a) * hkv + g) * D + ks * 16 + hf * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[ks][e] = static_cast<__bf16>(0.f);
    }
  }
  const bf16_t* Qg = static_cast<const bf16_t*>(a.q);
  const float cs = a.scale_log2;
  for (int qs = 0; qs < nqv; qs += kMQS) {
    const int qe = min(nqv, qs + kMQS);
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
        const int pos = a.pos0[r] + qv / a.G;
        const int lim = min(pos, T - 1) - (key0 + 32 * w + 4 * hf);
        float sv[16];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sv[i] = 8 * (i >> 2) + (i & 3) <= lim ? s[j][i] * cs : -INFINITY;
          m = fmaxf(m, sv[i]);
        }
        m = fmaxf(m, __shfl_xor(m, 32, kWave));
        float l = 0.f;
        if (m > -INFINITY) {
#pragma unroll
          for (int i = 0; i < 16; ++i) l += __builtin_amdgcn_exp2f(sv[i] - m);
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
  const int nqv = a.nq[r] * a.G;
  float colsum = 0.f;
  for (int q0 = 0; q0 < nqv; q0 += kMQB) {
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
  if (hf == 0 && kvalid)
    a.part[static_cast<int64_t>(g) * a.b.cu_N[a.b.n_req] + a.b.cu_N[r] + key] = colsum;
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
                                                       int n, float* __restrict__ scores) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int g = 0; g < hkv; ++g) s += part[static_cast<int64_t>(g) * n + i];
  scores[i] = s;
}

namespace {
struct MassLayout {
  int64_t rows;          // query rows used (sum over requests)
  int n_splits;
  int split_keys;
  size_t off_pm, off_pl, off_lse, off_part, total;
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
    const int key_tiles = std::max(1, ceil_div(max_T, kAT));
    int splits = static_cast<int>(std::min<int64_t>(key_tiles, ceil_div(512, static_cast<int>(std::min<int64_t>(base, 512)))));
    splits = std::max(1, std::min(splits, 64));
    m.split_keys = ceil_div(key_tiles, splits) * kAT;
    m.n_splits = ceil_div(std::max(max_T, 1), m.split_keys);
  }
  const int64_t plane = m.rows * L.n_q_heads;
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  m.off_pm = 0;
  m.off_pl = align(m.off_pm + sizeof(float) * plane * m.n_splits);
  m.off_lse = align(m.off_pl + sizeof(float) * plane * m.n_splits);
  m.off_part = align(m.off_lse + sizeof(float) * plane);
  m.total = align(m.off_part + sizeof(float) * static_cast<size_t>(L.n_kv_heads) * B.cu_N[B.n_req]);
  return m;
}
}  // namespace

size_t attn_mass_workspace(const kvf_layer_desc& L, const BatchArgs& B, int n_last_q) {
  return mass_layout(L, B, n_last_q).total;
}

hipError_t launch_attn_mass(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                            const void* q_u, int n_last_q, float* scores, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  const MassLayout lay = mass_layout(L, B, n_last_q);
  if (ws_bytes < lay.total) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  float* pm = reinterpret_cast<float*>(base + lay.off_pm);
  float* pl = reinterpret_cast<float*>(base + lay.off_pl);
  float* lse2 = reinterpret_cast<float*>(base + lay.off_lse);
  float* part = reinterpret_cast<float*>(base + lay.off_part);
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
  const int n = B.cu_N[B.n_req];
  if (plane == 0) {
    // no query rows: every key gets zero mass
    if (n > 0) {
      hipLaunchKernelGGL(head_sum_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st, part, 0, n,
                         scores);
    }
    return hipGetLastError();
  }

  // pass 1: softmax statistics of the used query rows
  if (L.dtype == KVF_BF16) {
    const dim3 grid(lay.n_splits * m.hkv, B.n_req);
    if (L.head_dim == 128)
      hipLaunchKernelGGL(mass_stats_bf16_kernel<128>, grid, dim3(256), 0, st, m);
    else
      hipLaunchKernelGGL(mass_stats_bf16_kernel<64>, grid, dim3(256), 0, st, m);
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
  hipLaunchKernelGGL(lse_combine_kernel, dim3(ceil_div(static_cast<int>(plane), 256 / kWave)),
                     dim3(256), 0, st, pm, pl, lay.n_splits, plane, plane, lse2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // pass 2: normalised probabilities summed per context key and kv head
  if (n == 0) return hipSuccess;
  if (L.dtype == KVF_BF16) {
    const int64_t blocks = static_cast<int64_t>(m.total_ktiles) * m.hkv;
    if (L.head_dim == 128)
      hipLaunchKernelGGL(mass_colsum_bf16_kernel<128>, dim3(blocks), dim3(256), 0, st, m);
    else
      hipLaunchKernelGGL(mass_colsum_bf16_kernel<64>, dim3(blocks), dim3(256), 0, st, m);
  } else {
    const int64_t waves = static_cast<int64_t>(n) * m.hkv;
    hipLaunchKernelGGL(mass_colsum_f32_kernel, dim3(ceil_div(static_cast<int>(waves), 4)),
                       dim3(256), 0, st, m, L.head_dim);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_sum_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st, part, L.n_kv_heads,
                     n, scores);
  return hipGetLastError();
}

}  // namespace kvf
