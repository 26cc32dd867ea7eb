// S4: gathered-row Q/K/V projection with a RoPE epilogue.
//
// QCFuse page, section 2.1.3 (Eq. 6-7): only the selected positions P (plus
// the query suffix) get fresh K/V under the current order and positions.
// KVBoost page, section 3.1 (Eq. 1): k = W_K x, v = W_V x; section 3.2 (Eq. 3):
// queries and keys carry the rotation of their position.
//
// bf16 path: Y[m, n] = sum_k X[row_src[m], k] W[n, k] on MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).  Workgroup tile 128 x 128 x 64,
// 4 waves in a 2 x 2 layout, double-buffered LDS, one barrier per K step.
// Rows of X are gathered through row_src while they are staged (each row
// slice is a contiguous 128-byte read).  Each wave owns two 32-column groups
// that are RoPE partners (channel j and j + d/2 of the same head), so the
// rotation is applied in registers on the accumulators.  Only the column
// tiles of the requested outputs (Q, K, V mask) are launched.
//
// fp32 path: a plain LDS-tiled FMA kernel (the fp32 workloads are small
// correctness shapes; MFMA is reserved for the bf16 contractions).
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
};

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
constexpr int kBM = 128, kBN = 128, kBK = 64, kPadK = 8, kLdK = kBK + kPadK;

__global__ void __launch_bounds__(256) gemm_qkv_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kBM][kLdK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kBN][kLdK];

  int t = blockIdx.y;
  const int seg = segment_of(a.n_tiles, t);
  const int n0 = t * kBN;                       // first column inside the segment
  const int m0 = blockIdx.x * kBM;
  const int K = a.K;
  const bf16_t* X = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.w) + static_cast<int64_t>(a.seg_w_row0[seg] + n0) * K;

  const int tid = threadIdx.x;
  const int lr = tid >> 3;                      // 0..31
  const int lk = (tid & 7) * 8;                 // 0..56
  const bf16_t* aptr[4];
  bool aval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + lr + 32 * i;
    int64_t src = -1;
    if (m < a.M) src = a.row_src ? static_cast<int64_t>(a.row_src[m]) : m;
    aval[i] = src >= 0 && src < a.x_rows;
    aptr[i] = X + (aval[i] ? src : 0) * K + lk;
  }
  const bf16_t* bptr = W + static_cast<int64_t>(lr) * K + lk;

  u32x4_t ra[4], rb[4];
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = aval[i] ? *reinterpret_cast<const u32x4_t*>(aptr[i]) : zero4;
    rb[i] = *reinterpret_cast<const u32x4_t*>(bptr + static_cast<int64_t>(32 * i) * K);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<u32x4_t*>(&As[0][lr + 32 * i][lk]) = ra[i];
    *reinterpret_cast<u32x4_t*>(&Bs[0][lr + 32 * i][lk]) = rb[i];
  }
  __syncthreads();

  const int w = tid >> 6, lane = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const int hg = a.d / 64;                      // 32-column groups per half head
  const int ga = (wn % hg) + (wn / hg) * 2 * hg;
  const int gb = ga + hg;
  const int lrow = lane & 31, lk8 = (lane >> 5) * 8;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / kBK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t ko = static_cast<int64_t>(kt + 1) * kBK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = aval[i] ? *reinterpret_cast<const u32x4_t*>(aptr[i] + ko) : zero4;
        rb[i] = *reinterpret_cast<const u32x4_t*>(bptr + static_cast<int64_t>(32 * i) * K + ko);
      }
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8_t*>(&As[cur][wm * 64 + mi * 32 + lrow][kk * 16 + lk8]);
      bfr[0] = *reinterpret_cast<const bf16x8_t*>(&Bs[cur][ga * 32 + lrow][kk * 16 + lk8]);
      bfr[1] = *reinterpret_cast<const bf16x8_t*>(&Bs[cur][gb * 32 + lrow][kk * 16 + lk8]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4_t*>(&As[cur ^ 1][lr + 32 * i][lk]) = ra[i];
        *reinterpret_cast<u32x4_t*>(&Bs[cur ^ 1][lr + 32 * i][lk]) = rb[i];
      }
    }
    __syncthreads();
  }

  // epilogue: rotate (Q, K) and store bf16
  const bool rope = seg < 2;
  const int half = a.d >> 1;
  const int ld = a.seg_heads[seg] * a.d;
  bf16_t* out = static_cast<bf16_t*>(a.out[seg]);
  const int ca = n0 + ga * 32 + lrow;
  const int cb = n0 + gb * 32 + lrow;
  const int j = ca % a.d;                       // < d/2 by construction
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= a.M) continue;
      float va = acc[mi][0][r], vb = acc[mi][1][r];
      if (rope) {
        const int p = a.row_pos[row];
        if (p < 0 || p >= a.rope_n) continue;
        const float c = a.rope_cos[static_cast<int64_t>(p) * half + j];
        const float s = a.rope_sin[static_cast<int64_t>(p) * half + j];
        const float oa = va * c - vb * s;
        const float ob = vb * c + va * s;
        va = oa;
        vb = ob;
      }
      out[static_cast<int64_t>(row) * ld + ca] = f32_to_bf16(va);
      out[static_cast<int64_t>(row) * ld + cb] = f32_to_bf16(vb);
    }
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
    if (row >= a.M) continue;
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
    out[static_cast<int64_t>(row) * ld + head * d + j] = lo;
    out[static_cast<int64_t>(row) * ld + head * d + half + j] = hi;
  }
}

hipError_t launch_recompute(const kvf_layer_desc& L, const void* x, int64_t x_rows,
                            const int32_t* row_src, const int32_t* row_pos, int M, const void* w,
                            uint32_t mask, const float* rc, const float* rs, int rope_n, void* q,
                            void* k, void* v, hipStream_t st) {
  GemmArgs a{};
  a.x = x;
  a.x_rows = x_rows;
  a.row_src = row_src;
  a.row_pos = row_pos;
  a.M = M;
  a.w = w;
  a.K = L.hidden;
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
    int total = 0;
    for (int s = 0; s < 3; ++s) {
      const int cols = heads[s] * L.head_dim;
      if (cols % kBN != 0) return hipErrorInvalidValue;   // rejected on the host earlier
      a.n_tiles[s] = (mask & bits[s]) ? cols / kBN : 0;
      total += a.n_tiles[s];
    }
    if (L.hidden % kBK != 0 || total == 0 || total > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_qkv_bf16_kernel, dim3(ceil_div(M, kBM), total), dim3(256), 0, st, a);
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
