// RoPE tables, S1 re-position + stitch of per-chunk caches (dense and int8
// KIVI dequant-on-load), and the offline KIVI int8 encoder.
//
// QCFuse page, section 2.1.2 (Eq. 3-4): chunk caches are built in isolation
// with keys at chunk-local positions from zero; serving remaps keys to request
// positions and stitches values in the same token order.  KVBoost page,
// section 3.2 (Eq. 3): the correction is the delta rotation R^(pos0).
// KVBoost page, section 4.5 (Eq. 7): KIVI int8, keys per channel, values per
// token.
//
// All kernels here are HBM-bound streams: 16-byte vector loads/stores, one
// chunk tile per workgroup so the chunk descriptor and its rotation row are
// fetched once per tile.
#include "../kvf_common.h"

namespace kvf {

// ---------------------------------------------------------------------------
// rope table: cos/sin(p * theta_j) in fp64, stored fp32
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) rope_table_kernel(double base, int d, int n_pos,
                                                         float* __restrict__ cs,
                                                         float* __restrict__ sn) {
  const int half = d / 2;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(n_pos) * half) return;
  const int p = static_cast<int>(i / half);
  const int j = static_cast<int>(i % half);
  const double theta = pow(base, -2.0 * static_cast<double>(j) / static_cast<double>(d));
  double s, c;
  sincos(static_cast<double>(p) * theta, &s, &c);
  cs[i] = static_cast<float>(c);
  sn[i] = static_cast<float>(s);
}

hipError_t launch_rope_table(double base, int d, int n_pos, float* c, float* s, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(n_pos) * (d / 2);
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     base, d, n_pos, c, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// S1: re-position and stitch
// ---------------------------------------------------------------------------
constexpr int kRotRows = 16;      // tokens per workgroup tile

struct RotArgs {
  const kvf_chunk* chunks;
  const void* pool_k;
  const void* pool_v;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_min;
  const float* k_scale;
  const float* v_min;
  const float* v_scale;
  int n_pool_chunks;
  int64_t pool_rows;
  const float* rope_cos;
  const float* rope_sin;
  int rope_n;
  void* fused_k;
  void* fused_v;
  int64_t fused_rows;
  int hkv;
  int d;
};

__device__ __forceinline__ void decode8(const uint8_t* codes, const float* mn, const float* sc,
                                        float (&v)[8]) {
  const u32x2_t c = *reinterpret_cast<const u32x2_t*>(codes);
  const float4 m0 = *reinterpret_cast<const float4*>(mn);
  const float4 m1 = *reinterpret_cast<const float4*>(mn + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(sc);
  const float4 s1 = *reinterpret_cast<const float4*>(sc + 4);
  const float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
  const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t q = (c[i >> 2] >> (8 * (i & 3))) & 0xffu;
    v[i] = fmaf(static_cast<float>(q), s[i], m[i]);
  }
}

template <typename T, bool KIVI>
__global__ void __launch_bounds__(256) rerotate_kernel(RotArgs a) {
  const kvf_chunk ch = a.chunks[blockIdx.x];
  const int t0 = blockIdx.y * kRotRows;
  if (ch.len <= 0 || t0 >= ch.len) return;
  // skip malformed descriptors instead of touching memory outside the buffers
  if (ch.src_row < 0 || static_cast<int64_t>(ch.src_row) + ch.len > a.pool_rows) return;
  if (ch.dst_row < 0 || static_cast<int64_t>(ch.dst_row) + ch.len > a.fused_rows) return;
  if (ch.pos0 < 0 || ch.pos0 >= a.rope_n) return;
  if (KIVI && (ch.pool_chunk < 0 || ch.pool_chunk >= a.n_pool_chunks)) return;

  const int d = a.d, half = d >> 1, hkv = a.hkv;
  const int row_elems = hkv * d;
  const int nrows = min(kRotRows, ch.len - t0);
  const float* cosr = a.rope_cos + static_cast<int64_t>(ch.pos0) * half;
  const float* sinr = a.rope_sin + static_cast<int64_t>(ch.pos0) * half;
  T* fk = static_cast<T*>(a.fused_k);
  T* fv = static_cast<T*>(a.fused_v);

  // keys: each unit rotates 8 low channels j0.. with their partners j0+half..
  const int kper = half >> 3;                 // units per head
  const int ku = hkv * kper;                  // units per token
  for (int u = threadIdx.x; u < nrows * ku; u += blockDim.x) {
    const int t = u / ku, w = u - t * ku;
    const int h = w / kper, j0 = (w - h * kper) << 3;
    const int64_t src = (static_cast<int64_t>(ch.src_row) + t0 + t) * row_elems + h * d;
    const int64_t dst = (static_cast<int64_t>(ch.dst_row) + t0 + t) * row_elems + h * d;
    float lo[8], hi[8];
    if constexpr (KIVI) {
      const int64_t st = (static_cast<int64_t>(ch.pool_chunk) * hkv + h) * d;
      decode8(a.k_codes + src + j0, a.k_min + st + j0, a.k_scale + st + j0, lo);
      decode8(a.k_codes + src + half + j0, a.k_min + st + half + j0, a.k_scale + st + half + j0, hi);
    } else {
      const T* pk = static_cast<const T*>(a.pool_k);
      Elem<T>::load8(pk + src + j0, lo);
      Elem<T>::load8(pk + src + half + j0, hi);
    }
    float c[8], s[8];
    Elem<float>::load8(cosr + j0, c);
    Elem<float>::load8(sinr + j0, s);
    float olo[8], ohi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      olo[i] = lo[i] * c[i] - hi[i] * s[i];
      ohi[i] = hi[i] * c[i] + lo[i] * s[i];
    }
    Elem<T>::store8(fk + dst + j0, olo);
    Elem<T>::store8(fk + dst + half + j0, ohi);
  }

  // values: stitched unchanged (decoded for int8 caches)
  const int vu = row_elems >> 3;
  for (int u = threadIdx.x; u < nrows * vu; u += blockDim.x) {
    const int t = u / vu, e0 = (u - t * vu) << 3;
    const int64_t srow = static_cast<int64_t>(ch.src_row) + t0 + t;
    const int64_t src = srow * row_elems + e0;
    const int64_t dst = (static_cast<int64_t>(ch.dst_row) + t0 + t) * row_elems + e0;
    float v[8];
    if constexpr (KIVI) {
      const int h = e0 / d;
      const float m = a.v_min[srow * hkv + h];
      const float sc = a.v_scale[srow * hkv + h];
      const u32x2_t cq = *reinterpret_cast<const u32x2_t*>(a.v_codes + src);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = fmaf(static_cast<float>((cq[i >> 2] >> (8 * (i & 3))) & 0xffu), sc, m);
    } else {
      Elem<T>::load8(static_cast<const T*>(a.pool_v) + src, v);
    }
    Elem<T>::store8(fv + dst, v);
  }
}

hipError_t launch_rerotate(const kvf_layer_desc& L, const kvf_chunk* chunks, int n_chunks,
                           int max_len, const void* pk, const void* pv, const kvf_kivi8* q,
                           int64_t pool_rows, const float* rc, const float* rs, int rope_n,
                           void* fk, void* fv, int64_t fused_rows, hipStream_t st) {
  RotArgs a{};
  a.chunks = chunks;
  a.pool_k = pk;
  a.pool_v = pv;
  if (q) {
    a.k_codes = q->k_codes;
    a.v_codes = q->v_codes;
    a.k_min = q->k_min;
    a.k_scale = q->k_scale;
    a.v_min = q->v_min;
    a.v_scale = q->v_scale;
    a.n_pool_chunks = q->n_pool_chunks;
  }
  a.pool_rows = pool_rows;
  a.rope_cos = rc;
  a.rope_sin = rs;
  a.rope_n = rope_n;
  a.fused_k = fk;
  a.fused_v = fv;
  a.fused_rows = fused_rows;
  a.hkv = L.n_kv_heads;
  a.d = L.head_dim;
  const dim3 grid(n_chunks, ceil_div(max_len, kRotRows));
  if (grid.y > 65535) return hipErrorInvalidValue;
  if (q)
    hipLaunchKernelGGL((rerotate_kernel<bf16_t, true>), grid, dim3(256), 0, st, a);
  else if (L.dtype == KVF_BF16)
    hipLaunchKernelGGL((rerotate_kernel<bf16_t, false>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((rerotate_kernel<float, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// offline KIVI int8 encoder (not on the fused-layer path)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint8_t kivi_code(float x, float mn, float inv) {
  const float t = (x - mn) * inv;
  return static_cast<uint8_t>(fminf(fmaxf(rintf(t), 0.f), 255.f));
}

// keys: one thread per (pool chunk, head, channel); two passes over the chunk
__global__ void __launch_bounds__(256) kivi_keys_kernel(const bf16_t* __restrict__ pk,
                                                        const int32_t* __restrict__ pool_cu,
                                                        int n_pool, int64_t pool_rows, int hkv,
                                                        int d, uint8_t* __restrict__ codes,
                                                        float* __restrict__ kmin,
                                                        float* __restrict__ kscale) {
  const int c = blockIdx.y;
  const int ch = blockIdx.x * blockDim.x + threadIdx.x;   // head * d + channel
  if (c >= n_pool || ch >= hkv * d) return;
  const int a = pool_cu[c], b = pool_cu[c + 1];
  if (a < 0 || b < a || b > pool_rows) return;
  const int row = hkv * d;
  float mn = INFINITY, mx = -INFINITY;
  for (int t = a; t < b; ++t) {
    const float x = bf16_to_f32(pk[static_cast<int64_t>(t) * row + ch]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  float sc = 0.f, inv = 0.f;
  if (b > a) {
    const float rng = mx - mn;
    if (rng > 0.f) {
      sc = rng / 255.f;
      inv = 255.f / rng;
    }
  } else {
    mn = 0.f;
  }
  kmin[static_cast<int64_t>(c) * row + ch] = mn;
  kscale[static_cast<int64_t>(c) * row + ch] = sc;
  for (int t = a; t < b; ++t) {
    const int64_t i = static_cast<int64_t>(t) * row + ch;
    codes[i] = kivi_code(bf16_to_f32(pk[i]), mn, inv);
  }
}

// values: one wave per (row, head)
__global__ void __launch_bounds__(256) kivi_values_kernel(const bf16_t* __restrict__ pv,
                                                          int64_t n_groups, int d,
                                                          uint8_t* __restrict__ codes,
                                                          float* __restrict__ vmin,
                                                          float* __restrict__ vscale) {
  const int64_t g = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (g >= n_groups) return;
  const bf16_t* src = pv + g * d;
  float mn = INFINITY, mx = -INFINITY;
  for (int j = lane; j < d; j += kWave) {
    const float x = bf16_to_f32(src[j]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  const float rng = mx - mn;
  const float sc = rng > 0.f ? rng / 255.f : 0.f;
  const float inv = rng > 0.f ? 255.f / rng : 0.f;
  if (lane == 0) {
    vmin[g] = mn;
    vscale[g] = sc;
  }
  for (int j = lane; j < d; j += kWave) codes[g * d + j] = kivi_code(bf16_to_f32(src[j]), mn, inv);
}

hipError_t launch_kivi8_encode(const kvf_layer_desc& L, const void* pk, const void* pv,
                               const int32_t* pool_cu, int n_pool, int64_t pool_rows, int max_len,
                               const kvf_kivi8& out, hipStream_t st) {
  (void)max_len;
  const int hkv = L.n_kv_heads, d = L.head_dim;
  if (n_pool > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kivi_keys_kernel, dim3(ceil_div(hkv * d, 256), n_pool), dim3(256), 0, st,
                     static_cast<const bf16_t*>(pk), pool_cu, n_pool, pool_rows, hkv, d,
                     const_cast<uint8_t*>(out.k_codes), const_cast<float*>(out.k_min),
                     const_cast<float*>(out.k_scale));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t groups = pool_rows * hkv;
  const int64_t blocks = (groups * kWave + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kivi_values_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(pv), groups, d, const_cast<uint8_t*>(out.v_codes),
                     const_cast<float*>(out.v_min), const_cast<float*>(out.v_scale));
  return hipGetLastError();
}

}  // namespace kvf
