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
//    O^T += V^T P^T directly from registers: the K dimension of that MFMA is
//    permuted to match the accumulator layout, and V is staged in LDS in a
//    4-key interleaved layout so each lane reads 4 consecutive keys of one
//    channel with one 8-byte LDS read.
//  * The causal mask uses each row's own position; keys beyond the tile's
//    last position are never loaded.
// The mass score runs the same loop in "statistics only" mode over key
// splits (pass 1: per-row log-sum-exp), combines the splits, then a second
// MFMA pass (S = Q K^T, query vectors on the MFMA rows) sums the normalised
// probabilities per key lane-locally and a last pass adds the kv heads in a
// fixed order, so the result is deterministic.
//
// fp32 path: one wave per (row, head) with lane-parallel keys; used by the
// small fp32 workloads only.
#include "../kvf_common.h"

namespace kvf {

constexpr int kAK = 64;          // keys per LDS tile
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
  int split_keys;                // keys per split (multiple of kAK)
  int hq, hkv, G;
  float scale_log2;
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int D, bool STATS_ONLY>
__global__ void __launch_bounds__(256) attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D / 16;       // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;       // 32-channel output blocks
  constexpr int LDK = D + 8;       // padded K row (bf16)
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kAK][LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[kAK / 4][D][4];
  __shared__ int s_maxpos;

  const int hkv = a.hkv;
  const int g = blockIdx.x % hkv;
  const int tile = a.total_tiles - 1 - static_cast<int>(blockIdx.x / hkv);
  const int r = find_segment(a.cu_tiles, a.b.n_req, tile);
  const int tr = tile - a.cu_tiles[r];
  const int R = a.rows_per_tile;
  const int lrow0 = tr * R;                               // first row inside the request
  const int nrows = min(R, a.nrows[r] - lrow0);
  const int T = a.b.cu_T[r + 1] - a.b.cu_T[r];
  const int64_t krow0 = a.b.cu_T[r];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, hf = lane >> 5;
  const int qv = 32 * w + c;
  const int row_l = qv % R, head_l = qv / R;
  const bool valid = head_l < a.G && row_l < nrows;
  const int64_t qrow = static_cast<int64_t>(a.qrow0[r]) + lrow0 + row_l;
  const int h = g * a.G + head_l;
  int pos = -1;
  if (valid) {
    pos = a.q_pos ? a.q_pos[qrow] : a.pos0[r] + lrow0 + row_l;
    if (pos < 0 || pos >= T) pos = -1;
  }
  if (tid == 0) s_maxpos = -1;
  __syncthreads();
  if (pos >= 0) atomicMax(&s_maxpos, pos);
  __syncthreads();
  const int kend = s_maxpos + 1;                           // keys [0, kend) are visible to someone

  int kbeg = 0, klim = kend;
  if constexpr (STATS_ONLY) {
    kbeg = blockIdx.y * a.split_keys;
    klim = min(kend, kbeg + a.split_keys);
  }

  // Q fragments (B operand of S^T = K Q^T): channel chunk ks*16 + hf*8
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
  if constexpr (!STATS_ONLY) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  const bf16_t* Kg = static_cast<const bf16_t*>(a.k);
  const bf16_t* Vg = static_cast<const bf16_t*>(a.v);
  constexpr int VPR = D / 8;                              // 16-byte vectors per key row
  for (int kb0 = kbeg; kb0 < klim; kb0 += kAK) {
    __syncthreads();
    for (int idx = tid; idx < kAK * VPR; idx += 256) {
      const int kr = idx / VPR, vc = idx - kr * VPR;
      const int key = kb0 + kr;
      u32x4_t kv4 = {0u, 0u, 0u, 0u}, vv4 = {0u, 0u, 0u, 0u};
      if (key < klim) {
        const int64_t off = ((krow0 + key) * hkv + g) * D + vc * 8;
        kv4 = *reinterpret_cast<const u32x4_t*>(Kg + off);
        if constexpr (!STATS_ONLY) vv4 = *reinterpret_cast<const u32x4_t*>(Vg + off);
      }
      *reinterpret_cast<u32x4_t*>(&Ks[kr][vc * 8]) = kv4;
      if constexpr (!STATS_ONLY) {
        const u16x8_t vh = __builtin_bit_cast(u16x8_t, vv4);
#pragma unroll
        for (int e = 0; e < 8; ++e) Vs[kr >> 2][vc * 8 + e][kr & 3] = vh[e];
      }
    }
    __syncthreads();

    // S^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t kfrag = *reinterpret_cast<const bf16x8_t*>(&Ks[kb * 32 + c][ks * 16 + hf * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // scale, mask, tile max
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb0 + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
        const float v = (key <= pos && key < klim) ? s[kb][i] * a.scale_log2 : -INFINITY;
        s[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = exp2f(s[kb][i] - m_use);
        // the V product consumes bf16 probabilities: normalise by the sum of
        // exactly those values so the weights used sum to one
        if constexpr (!STATS_ONLY) p = static_cast<float>(static_cast<__bf16>(p));
        s[kb][i] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32, kWave);
    l_run = l_run * alpha + rs;
    m_run = m_new;

    if constexpr (!STATS_ONLY) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bf16x8_t pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[kb][8 * st + e]);
          const int key_a = kb * 32 + 16 * st + 4 * hf;  // keys key_a..+3 and key_a+8..+11
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u16x4_t lo = *reinterpret_cast<const u16x4_t*>(&Vs[key_a >> 2][db * 32 + c][0]);
            const u16x4_t hi = *reinterpret_cast<const u16x4_t*>(&Vs[(key_a + 8) >> 2][db * 32 + c][0]);
            const u16x8_t vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pb,
                                                            o[db], 0, 0, 0);
          }
        }
      }
    }
  }

  if (!valid || pos < 0) return;
  const int64_t orow = static_cast<int64_t>(a.orow0[r]) + lrow0 + row_l;
  if constexpr (STATS_ONLY) {
    if (hf == 0) {
      const int64_t idx = static_cast<int64_t>(blockIdx.y) * a.plane + orow * a.hq + h;
      a.part_m[idx] = m_run;
      a.part_l[idx] = l_run;
    }
  } else {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16_t* O = static_cast<bf16_t*>(a.out) + (orow * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * hf;
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv);
        pk[1] = pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
        *reinterpret_cast<u32x2_t*>(O + d0) = pk;
      }
    if (a.lse && hf == 0) a.lse[orow * a.hq + h] = (m_run + log2f(l_run)) * kLn2;
  }
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
    if (L.head_dim == 128)
      hipLaunchKernelGGL((attn_bf16_kernel<128, false>), dim3(blocks), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<64, false>), dim3(blocks), dim3(256), 0, st, a);
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
// combine split statistics into log2-domain LSE per (row, head)
__global__ void __launch_bounds__(256) lse_combine_kernel(const float* __restrict__ pm,
                                                          const float* __restrict__ pl, int n_splits,
                                                          int64_t plane, int64_t n,
                                                          float* __restrict__ lse2) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float m = -INFINITY;
  for (int s = 0; s < n_splits; ++s) m = fmaxf(m, pm[s * plane + i]);
  float l = 0.f;
  if (m > -INFINITY)
    for (int s = 0; s < n_splits; ++s) {
      const float ms = pm[s * plane + i];
      if (ms > -INFINITY) l += pl[s * plane + i] * exp2f(ms - m);
    }
  lse2[i] = l > 0.f ? m + log2f(l) : INFINITY;     // INFINITY: row contributes nothing
}

struct MassArgs {
  BatchArgs b;
  int qrow0[KVF_MAX_REQ];        // first q_u row used by each request
  int nq[KVF_MAX_REQ];           // query rows used
  int orow0[KVF_MAX_REQ];        // their rows in lse2
  int cu_ktiles[KVF_MAX_REQ + 1];
  int total_ktiles;
  const void* q;
  const void* k;
  const float* lse2;             // [rows, Hq]
  float* part;                   // [Hkv, sum N]
  int hq, hkv, G;
  float scale_log2;
};

constexpr int kMK = 128;         // context keys per workgroup (4 waves x 32)

template <int D>
__global__ void __launch_bounds__(256) mass_colsum_bf16_kernel(MassArgs a) {
  constexpr int KS = D / 16;
  constexpr int LDQ = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[32][LDQ];
  __shared__ float Ls[32];
  const int g = blockIdx.x % a.hkv;
  const int kt = static_cast<int>(blockIdx.x / a.hkv);
  const int r = find_segment(a.cu_ktiles, a.b.n_req, kt);
  const int key0 = (kt - a.cu_ktiles[r]) * kMK;
  const int N = a.b.n_ctx[r];
  const int64_t krow0 = a.b.cu_T[r];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  constexpr int VPR = D / 8;
  for (int q0 = 0; q0 < nqv; q0 += 32) {
    __syncthreads();
    for (int idx = tid; idx < 32 * VPR; idx += 256) {
      const int qq = idx / VPR, vc = idx - qq * VPR;
      const int qi = q0 + qq;
      u32x4_t v4 = {0u, 0u, 0u, 0u};
      if (qi < nqv) {
        const int row = qi / a.G, hl = qi - row * a.G;
        v4 = *reinterpret_cast<const u32x4_t*>(
            Qg + ((static_cast<int64_t>(a.qrow0[r]) + row) * a.hq + g * a.G + hl) * D + vc * 8);
      }
      *reinterpret_cast<u32x4_t*>(&Qs[qq][vc * 8]) = v4;
    }
    if (tid < 32) {
      const int qi = q0 + tid;
      float l2 = INFINITY;
      if (qi < nqv) {
        const int row = qi / a.G, hl = qi - row * a.G;
        l2 = a.lse2[(static_cast<int64_t>(a.orow0[r]) + row) * a.hq + g * a.G + hl];
      }
      Ls[tid] = l2;
    }
    __syncthreads();
    f32x16_t s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t qfrag = *reinterpret_cast<const bf16x8_t*>(&Qs[c][ks * 16 + hf * 8]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfrag, kf[ks], s, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qq = 8 * (i >> 2) + 4 * hf + (i & 3);
      colsum += exp2f(s[i] * a.scale_log2 - Ls[qq]);    // Ls = +inf for padding rows -> 0
    }
  }
  colsum += __shfl_xor(colsum, 32, kWave);
  if (hf == 0 && kvalid) a.part[static_cast<int64_t>(g) * a.b.cu_N[a.b.n_req] + a.b.cu_N[r] + key] = colsum;
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
  int64_t tiles = 0;
  const int G = L.n_q_heads / L.n_kv_heads;
  const int R = L.dtype == KVF_BF16 ? rows_per_tile(G) : 1;
  for (int r = 0; r < B.n_req; ++r) {
    const int U = B.cu_T[r + 1] - B.cu_T[r] - B.n_ctx[r];
    const int nq = n_last_q > 0 ? std::min(n_last_q, U) : U;
    m.rows += nq;
    tiles += ceil_div(nq, R);
    max_T = std::max(max_T, B.cu_T[r + 1] - B.cu_T[r]);
  }
  // enough workgroups in the statistics pass to cover the chip twice
  const int64_t base = std::max<int64_t>(1, L.dtype == KVF_BF16 ? tiles * L.n_kv_heads
                                                                : m.rows * L.n_q_heads / 4);
  const int key_tiles = std::max(1, ceil_div(max_T, kAK));
  int splits = static_cast<int>(std::min<int64_t>(key_tiles, ceil_div(512, static_cast<int>(std::min<int64_t>(base, 512)))));
  splits = std::max(1, std::min(splits, 64));
  m.split_keys = ceil_div(key_tiles, splits) * kAK;
  m.n_splits = ceil_div(std::max(max_T, 1), m.split_keys);
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

  // pass 1: per-split softmax statistics of the used query rows
  AttnArgs a{};
  a.b = B;
  int orow = 0;
  for (int r = 0; r < B.n_req; ++r) {
    const int U = B.cu_T[r + 1] - B.cu_T[r] - B.n_ctx[r];
    const int nq = n_last_q > 0 ? std::min(n_last_q, U) : U;
    a.qrow0[r] = B.cu_U[r] + (U - nq);
    a.nrows[r] = nq;
    a.pos0[r] = B.n_ctx[r] + (U - nq);
    a.orow0[r] = orow;
    orow += nq;
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
  if (plane > 0) {
    if (L.dtype == KVF_BF16) {
      fill_tiles(a, rows_per_tile(G));
      const dim3 grid(a.total_tiles * a.hkv, lay.n_splits);
      if (L.head_dim == 128)
        hipLaunchKernelGGL((attn_bf16_kernel<128, true>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, dim3(256), 0, st, a);
    } else {
      const dim3 grid(ceil_div(static_cast<int>(plane), 4), lay.n_splits);
      hipLaunchKernelGGL((attn_f32_kernel<true>), grid, dim3(256), 0, st, a, L.head_dim,
                         static_cast<int>(lay.rows));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lse_combine_kernel, dim3(ceil_div(static_cast<int>(plane), 256)), dim3(256),
                       0, st, pm, pl, lay.n_splits, plane, plane, lse2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  // pass 2: normalised probabilities summed per context key and kv head
  MassArgs m{};
  m.b = B;
  for (int r = 0; r < B.n_req; ++r) {
    m.qrow0[r] = a.qrow0[r];
    m.nq[r] = a.nrows[r];
    m.orow0[r] = a.orow0[r];
    m.cu_ktiles[r + 1] = m.cu_ktiles[r] + ceil_div(B.n_ctx[r], kMK);
  }
  m.total_ktiles = m.cu_ktiles[B.n_req];
  m.q = q_u;
  m.k = fk;
  m.lse2 = lse2;
  m.part = part;
  m.hq = L.n_q_heads;
  m.hkv = L.n_kv_heads;
  m.G = G;
  m.scale_log2 = scale_log2;
  const int n = B.cu_N[B.n_req];
  if (L.dtype == KVF_BF16) {
    const int64_t blocks = static_cast<int64_t>(m.total_ktiles) * m.hkv;
    if (L.head_dim == 128)
      hipLaunchKernelGGL(mass_colsum_bf16_kernel<128>, dim3(blocks), dim3(256), 0, st, m);
    else
      hipLaunchKernelGGL(mass_colsum_bf16_kernel<64>, dim3(blocks), dim3(256), 0, st, m);
  } else {
    const int64_t waves = static_cast<int64_t>(n) * m.hkv;
    hipLaunchKernelGGL(mass_colsum_f32_kernel, dim3(ceil_div(static_cast<int>(waves), 4)), dim3(256),
                       0, st, m, L.head_dim);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_sum_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st, part, L.n_kv_heads,
                     n, scores);
  return hipGetLastError();
}

}  // namespace kvf
