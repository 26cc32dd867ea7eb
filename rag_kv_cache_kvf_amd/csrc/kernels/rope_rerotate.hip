// RoPE tables, S1 re-position + stitch of per-chunk caches (dense, and KIVI
// int8 / int4 dequant-on-load) into a bf16 or an int8-resident fused cache,
// and the offline KIVI encoder.
//
// QCFuse page, section 2.1.2 (Eq. 3-4): chunk caches are built in isolation
// with keys at chunk-local positions from zero; serving remaps keys to request
// positions and stitches values in the same token order.  KVBoost page,
// section 3.2 (Eq. 3): the correction is the delta rotation R^(pos0).
// KVBoost page, section 4.5 (Eq. 7): KIVI with b = 8 or 4 bits, keys per
// channel, values per token; 4-bit codes two to a byte, channel 2i in the
// low nibble.
//
// All kernels here are HBM-bound streams: 16-byte vector loads/stores, one
// chunk tile per workgroup so the chunk descriptor and its rotation row are
// fetched once per tile.  In keys-only mode the values were stitched by the
// loader and are not touched; the keys may be rotated in place (a thread
// reads the 16 channels of a rotation pair set before it writes them).
#include <algorithm>
#include <type_traits>

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
constexpr int kRotRows = 8;       // tokens per workgroup tile (at least; see rot_rows)

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
  int k_only;                     // keys only: values are already in place
  int rows;                       // tokens per workgroup tile
  // Deviation score of the re-positioned keys in the same pass (S2b fused
  // into S1): k_fresh [fused rows, Hkv, d] in T, rows indexed like the fused
  // cache; the score of a context row of request r goes to entry
  // cu_N[r] + (row - cu_T[r]) of dev.scores.  Unused unless the kernel's
  // DEV parameter is set.
  const void* k_fresh;
  ScoreOut dev;
  BatchArgs B;
};

// Tokens per workgroup tile: kRotRows, or more when a token's key has too
// few rotation units (Hkv d / 16) for the tile to give each of the 256
// threads one (narrow rows: Hkv = 2, d = 128 takes 16 tokens).
static int rot_rows(int hkv, int d, bool kivi) {
  const int ku = std::max(1, hkv * d / 16);
  const int rows = std::max(kRotRows, ceil_div(256, ku));
  // KIVI: each thread reuses its unit's statistics over 4 rows
  return kivi ? 4 * rows : rows;
}

// the 8 codes of channels e..e+7 (e a multiple of 8), `codes` pointing at
// their first byte: 8 bytes for b = 8, 4 bytes for b = 4 (channel i of the
// eight in bits 4i..4i+3 of the little-endian word)
template <int BITS>
__device__ __forceinline__ void codes8(const uint8_t* codes, uint32_t (&q)[8]) {
  if constexpr (BITS == 8) {
    const u32x2_t c = *reinterpret_cast<const u32x2_t*>(codes);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (c[i >> 2] >> (8 * (i & 3))) & 0xffu;
  } else {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(codes);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (c >> (4 * i)) & 0xfu;
  }
}

template <int BITS>
__device__ __forceinline__ void decode8(const uint8_t* codes, const float* mn, const float* sc,
                                        float (&v)[8]) {
  uint32_t q[8];
  codes8<BITS>(codes, q);
  const float4 m0 = *reinterpret_cast<const float4*>(mn);
  const float4 m1 = *reinterpret_cast<const float4*>(mn + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(sc);
  const float4 s1 = *reinterpret_cast<const float4*>(sc + 4);
  const float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
  const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fmaf(static_cast<float>(q[i]), s[i], m[i]);
}

// 8 consecutive floats (16-byte aligned)
__device__ __forceinline__ void load8f(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One RoPE pair (x, y) rotated by (c, s): (x c - y s, y c + x s), with the
// multiply-adds spelled out so that every instantiation of a kernel rounds
// the same way (left to the compiler, the contraction into fused
// multiply-adds may differ between instantiations and change the last bit).
__device__ __forceinline__ float rot_lo(float x, float y, float c, float s) {
  return fmaf(x, c, -(y * s));
}
__device__ __forceinline__ float rot_hi(float x, float y, float c, float s) {
  return fmaf(y, c, x * s);
}

// a value as the fused cache stores it (bf16: rounded to nearest even)
template <typename T>
__device__ __forceinline__ float stored(float x) {
  if constexpr (std::is_same_v<T, float>) return x;
  else return bf16_to_f32(f32_to_bf16(x));
}

// Deviation score of fused row `frow` (KVBoost page, section 4.6.2,
// Algorithm 2 at one layer): 1 - (1/Hkv) sum_h cos(k_fused[h], k_fresh[h]),
// a head's cosine 0 when either norm is 0, from the key as the fused cache
// stores it.  The row's rotation units sit on ku consecutive lanes (ku a
// power of two dividing 64), kper per head, and all of them call this
// together; this lane holds channels j0.. and their partners half + j0.. of
// head h.  Rows that are not context rows of the batch get no score.
template <typename T>
__device__ __forceinline__ void deviation_of_row(const RotArgs& a, int64_t frow, int h, int j0,
                                                 const float (&lo)[8], const float (&hi)[8],
                                                 int ku, int kper) {
  const BatchArgs& B = a.B;
  const int half = a.d >> 1;
  bool ctx = frow < B.cu_T[B.n_req];
  int64_t j = 0;
  if (ctx) {
    const int r = find_segment(B.cu_T, B.n_req, static_cast<int>(frow));
    const int64_t i = frow - B.cu_T[r];
    ctx = i < B.n_ctx[r];
    j = B.cu_N[r] + i;
  }
  float dot = 0.f, nx = 0.f, ny = 0.f;
  if (ctx && score_eligible(a.dev, j)) {       // ineligible rows' k_fresh is not read
    const T* kf = static_cast<const T*>(a.k_fresh) + (frow * a.hkv + h) * a.d;
    float ylo[8], yhi[8];
    Elem<T>::load8(kf + j0, ylo);
    Elem<T>::load8(kf + half + j0, yhi);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xl = stored<T>(lo[i]), xh = stored<T>(hi[i]);
      dot = fmaf(xl, ylo[i], fmaf(xh, yhi[i], dot));
      nx = fmaf(xl, xl, fmaf(xh, xh, nx));
      ny = fmaf(ylo[i], ylo[i], fmaf(yhi[i], yhi[i], ny));
    }
  }
  dot = group_sum(dot, kper);
  nx = group_sum(nx, kper);
  ny = group_sum(ny, kper);
  const int lane = threadIdx.x & (kWave - 1);
  const float den = sqrtf(nx) * sqrtf(ny);
  float c = ((lane & (kper - 1)) == 0 && den > 0.f) ? dot / den : 0.f;
  c = group_sum(c, ku);
  if ((lane & (ku - 1)) == 0 && ctx) store_score(a.dev, j, 1.f - c / static_cast<float>(a.hkv));
}

// KB: 0 for a dense cache in T, else the KIVI code width (8 or 4).
// DEV: also the deviation score of every re-positioned context row.
template <typename T, int KB, bool DEV>
__global__ void __launch_bounds__(256) rerotate_kernel(RotArgs a) {
  constexpr bool KIVI = KB != 0;
  const kvf_chunk ch = a.chunks[blockIdx.x];
  const int t0 = blockIdx.y * a.rows;
  if (ch.len <= 0 || t0 >= ch.len) return;
  // skip malformed descriptors instead of touching memory outside the buffers
  if (ch.src_row < 0 || static_cast<int64_t>(ch.src_row) + ch.len > a.pool_rows) return;
  if (ch.dst_row < 0 || static_cast<int64_t>(ch.dst_row) + ch.len > a.fused_rows) return;
  if (ch.pos0 < 0 || ch.pos0 >= a.rope_n) return;
  if (KIVI && (ch.pool_chunk < 0 || ch.pool_chunk >= a.n_pool_chunks)) return;

  const int d = a.d, half = d >> 1, hkv = a.hkv;
  const int row_elems = hkv * d;
  const int nrows = min(a.rows, ch.len - t0);
  const float* cosr = a.rope_cos + static_cast<int64_t>(ch.pos0) * half;
  const float* sinr = a.rope_sin + static_cast<int64_t>(ch.pos0) * half;
  T* fk = static_cast<T*>(a.fused_k);
  T* fv = static_cast<T*>(a.fused_v);

  // keys: each unit rotates 8 low channels j0.. with their partners j0+half..
  const int kper = half >> 3;                 // units per head
  const int ku = hkv * kper;                  // units per token
  if (KIVI && blockDim.x % ku == 0) {
    // a thread keeps one unit (head, channels) over the tile's rows, so the
    // chunk's per-channel key statistics and the rotation factors are read
    // once per thread instead of once per row
    const int w = threadIdx.x % ku;
    const int h = w / kper, j0 = (w - h * kper) << 3;
    const int64_t st = (static_cast<int64_t>(ch.pool_chunk) * hkv + h) * d;
    float mlo[8], slo[8], mhi[8], shi[8], c[8], s[8];
    load8f(a.k_min + st + j0, mlo);
    load8f(a.k_scale + st + j0, slo);
    load8f(a.k_min + st + half + j0, mhi);
    load8f(a.k_scale + st + half + j0, shi);
    load8f(cosr + j0, c);
    load8f(sinr + j0, s);
    for (int t = threadIdx.x / ku; t < nrows; t += blockDim.x / ku) {
      const int64_t src = (static_cast<int64_t>(ch.src_row) + t0 + t) * row_elems + h * d;
      const int64_t dst = (static_cast<int64_t>(ch.dst_row) + t0 + t) * row_elems + h * d;
      uint32_t qlo[8], qhi[8];
      codes8<KIVI ? KB : 8>(a.k_codes + (src + j0) * KB / 8, qlo);
      codes8<KIVI ? KB : 8>(a.k_codes + (src + half + j0) * KB / 8, qhi);
      float olo[8], ohi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float lo = fmaf(static_cast<float>(qlo[i]), slo[i], mlo[i]);
        const float hi = fmaf(static_cast<float>(qhi[i]), shi[i], mhi[i]);
        olo[i] = rot_lo(lo, hi, c[i], s[i]);
        ohi[i] = rot_hi(lo, hi, c[i], s[i]);
      }
      Elem<T>::store8(fk + dst + j0, olo);
      Elem<T>::store8(fk + dst + half + j0, ohi);
      if constexpr (DEV)
        deviation_of_row<T>(a, static_cast<int64_t>(ch.dst_row) + t0 + t, h, j0, olo, ohi, ku, kper);
    }
  } else
  for (int u = threadIdx.x; u < nrows * ku; u += blockDim.x) {
    const int t = u / ku, w = u - t * ku;
    const int h = w / kper, j0 = (w - h * kper) << 3;
    const int64_t src = (static_cast<int64_t>(ch.src_row) + t0 + t) * row_elems + h * d;
    const int64_t dst = (static_cast<int64_t>(ch.dst_row) + t0 + t) * row_elems + h * d;
    float lo[8], hi[8];
    if constexpr (KIVI) {
      const int64_t st = (static_cast<int64_t>(ch.pool_chunk) * hkv + h) * d;
      decode8<KB>(a.k_codes + (src + j0) * KB / 8, a.k_min + st + j0, a.k_scale + st + j0, lo);
      decode8<KB>(a.k_codes + (src + half + j0) * KB / 8, a.k_min + st + half + j0,
                  a.k_scale + st + half + j0, hi);
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
      olo[i] = rot_lo(lo[i], hi[i], c[i], s[i]);
      ohi[i] = rot_hi(lo[i], hi[i], c[i], s[i]);
    }
    Elem<T>::store8(fk + dst + j0, olo);
    Elem<T>::store8(fk + dst + half + j0, ohi);
    if constexpr (DEV)
      deviation_of_row<T>(a, static_cast<int64_t>(ch.dst_row) + t0 + t, h, j0, olo, ohi, ku, kper);
  }

  // values: stitched unchanged (decoded for int8 caches)
  if (!KIVI && a.k_only) return;
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
      uint32_t q[8];
      codes8<KB>(a.v_codes + src * KB / 8, q);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = fmaf(static_cast<float>(q[i]), sc, m);
    } else {
      Elem<T>::load8(static_cast<const T*>(a.pool_v) + src, v);
    }
    Elem<T>::store8(fv + dst, v);
  }
}

// Rotation units of one fused row (8 channel pairs each) when the fused
// deviation score can reduce a row within aligned lane groups: a power of
// two dividing 64, else 0.
int rerotate_deviation_lanes(int hkv, int d) {
  const int ku = hkv * d / 16;
  return (d % 16 == 0 && ku >= 1 && ku <= kWave && (ku & (ku - 1)) == 0) ? ku : 0;
}

hipError_t launch_rerotate(const kvf_layer_desc& L, const kvf_chunk* chunks, int n_chunks,
                           int max_len, const void* pk, const void* pv, const kvf_kivi* q,
                           int64_t pool_rows, const float* rc, const float* rs, int rope_n,
                           void* fk, void* fv, int64_t fused_rows, int k_only, hipStream_t st,
                           const RotDeviation* dev) {
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
  a.k_only = k_only;
  a.rows = rot_rows(a.hkv, a.d, q != nullptr);
  const dim3 grid(n_chunks, ceil_div(max_len, a.rows));
  if (grid.y > 65535) return hipErrorInvalidValue;
  if (dev) {
    if (rerotate_deviation_lanes(a.hkv, a.d) == 0) return hipErrorInvalidValue;
    a.k_fresh = dev->k_fresh;
    a.dev = dev->out;
    a.B = dev->B;
  }
#define KVF_ROT_LAUNCH(T_, KB_)                                                               \
  do {                                                                                        \
    if (dev) hipLaunchKernelGGL((rerotate_kernel<T_, KB_, true>), grid, dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((rerotate_kernel<T_, KB_, false>), grid, dim3(256), 0, st, a);    \
  } while (0)
  if (q && q->bits == 4)
    KVF_ROT_LAUNCH(bf16_t, 4);
  else if (q)
    KVF_ROT_LAUNCH(bf16_t, 8);
  else if (L.dtype == KVF_BF16)
    KVF_ROT_LAUNCH(bf16_t, 0);
  else
    KVF_ROT_LAUNCH(float, 0);
#undef KVF_ROT_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// S1 into an int8-resident fused cache
// ---------------------------------------------------------------------------
// Work items are (row of a chunk, kv head), d/8 lanes each: lane j of an
// item takes the four rotation pairs (4j + i, 4j + i + d/2), i < 4, so its
// code bytes move as two 4-byte words, its statistics, cos and sin as float4
// loads, and the item's 8-bit group is encoded after one min/max reduction
// over its lanes.  A wave holds 8 (d = 128) or 16 (d = 64) items.
constexpr int kQ8RotWaves = 4;

struct RotQ8Args {
  const kvf_chunk* chunks;
  const bf16_t* pool_k;           // dense per-chunk cache
  const bf16_t* pool_v;
  const uint8_t* k_codes;         // 8-bit KIVI per-chunk cache
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
  kvf_q8_cache out;
  int hkv;
  int d;
  // deviation score of the re-positioned keys as the cache stores them
  // (kvf_rerotate_q8_deviation; unused unless the kernel's DEV is set)
  const bf16_t* k_fresh;          // [out.rows, Hkv, d]
  ScoreOut dev;
  BatchArgs B;
};

__device__ __forceinline__ void bytes4(uint32_t w, float (&x)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = static_cast<float>((w >> (8 * i)) & 0xffu);
}

// the 8 values of one lane -> 8 codes (two words, channels 4j.. and
// 4j + d/2..) and the item's (min, scale); `gl` lanes per item
__device__ __forceinline__ void encode8(const float (&lo)[4], const float (&hi)[4], int gl, bool valid,
                                        uint32_t& w_lo, uint32_t& w_hi, float& mn, float& sc) {
  mn = INFINITY;
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mn = fminf(mn, fminf(lo[i], hi[i]));
    mx = fmaxf(mx, fmaxf(lo[i], hi[i]));
  }
  if (!valid) {
    mn = INFINITY;
    mx = -INFINITY;
  }
  group_minmax(mn, mx, gl);
  float inv;
  kivi_stats<8>(mn, mx, sc, inv);
  w_lo = w_hi = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w_lo |= kivi_code<8>(lo[i], mn, inv) << (8 * i);
    w_hi |= kivi_code<8>(hi[i], mn, inv) << (8 * i);
  }
}

// KB: 0 for a dense bf16 per-chunk cache, 8 for an 8-bit KIVI one.
// DEV: also the deviation score of every re-positioned context row; the
// items of a row (its Hkv heads) then sit on Hkv * d / 8 consecutive lanes,
// a power of two dividing 64, and no row straddles two workgroups.
template <int KB, bool DEV>
__global__ void __launch_bounds__(64 * kQ8RotWaves) rerotate_q8_kernel(RotQ8Args a) {
  const kvf_chunk ch = a.chunks[blockIdx.x];
  if (ch.len <= 0) return;
  if (ch.src_row < 0 || static_cast<int64_t>(ch.src_row) + ch.len > a.pool_rows) return;
  if (ch.dst_row < 0 || static_cast<int64_t>(ch.dst_row) + ch.len > a.out.rows) return;
  if (ch.pos0 < 0 || ch.pos0 >= a.rope_n) return;
  if (KB && (ch.pool_chunk < 0 || ch.pool_chunk >= a.n_pool_chunks)) return;

  const int d = a.d, half = d >> 1, hkv = a.hkv;
  const int gl = d >> 3;                           // lanes per item
  const int ipb = kQ8RotWaves * kWave / gl;        // items per workgroup
  const int lane_in = threadIdx.x & (gl - 1);
  const int item = blockIdx.y * ipb + static_cast<int>(threadIdx.x) / gl;
  const int t = item / hkv, h = item - t * hkv;
  // items past the chunk take part in the reductions of their wave only
  const bool valid = t < ch.len;
  const int j = 4 * lane_in;                       // first channel of the low quad
  const int64_t srow = static_cast<int64_t>(ch.src_row) + (valid ? t : 0);
  const int64_t drow = static_cast<int64_t>(ch.dst_row) + (valid ? t : 0);
  const int64_t src = (srow * hkv + h) * d + j;    // element offset of channel j
  const int64_t dst = (drow * hkv + h) * d + j;
  // keys: decode, rotate by R(pos0), encode
  float lo[4] = {0.f, 0.f, 0.f, 0.f}, hi[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    if constexpr (KB == 8) {
      const int64_t st = (static_cast<int64_t>(ch.pool_chunk) * hkv + h) * d + j;
      float cl[4], chh[4];
      bytes4(*reinterpret_cast<const uint32_t*>(a.k_codes + src), cl);
      bytes4(*reinterpret_cast<const uint32_t*>(a.k_codes + src + half), chh);
      const float4 ml = *reinterpret_cast<const float4*>(a.k_min + st);
      const float4 sl = *reinterpret_cast<const float4*>(a.k_scale + st);
      const float4 mh = *reinterpret_cast<const float4*>(a.k_min + st + half);
      const float4 sh = *reinterpret_cast<const float4*>(a.k_scale + st + half);
      const float mlv[4] = {ml.x, ml.y, ml.z, ml.w}, slv[4] = {sl.x, sl.y, sl.z, sl.w};
      const float mhv[4] = {mh.x, mh.y, mh.z, mh.w}, shv[4] = {sh.x, sh.y, sh.z, sh.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = fmaf(cl[i], slv[i], mlv[i]);
        hi[i] = fmaf(chh[i], shv[i], mhv[i]);
      }
    } else {
      const u32x2_t wl = *reinterpret_cast<const u32x2_t*>(a.pool_k + src);
      const u32x2_t wh = *reinterpret_cast<const u32x2_t*>(a.pool_k + src + half);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        lo[2 * i] = __uint_as_float(wl[i] << 16);
        lo[2 * i + 1] = __uint_as_float(wl[i] & 0xffff0000u);
        hi[2 * i] = __uint_as_float(wh[i] << 16);
        hi[2 * i + 1] = __uint_as_float(wh[i] & 0xffff0000u);
      }
    }
  }
  const float4 c4 = *reinterpret_cast<const float4*>(a.rope_cos + static_cast<int64_t>(ch.pos0) * half + j);
  const float4 s4 = *reinterpret_cast<const float4*>(a.rope_sin + static_cast<int64_t>(ch.pos0) * half + j);
  const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
  float rlo[4], rhi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rlo[i] = rot_lo(lo[i], hi[i], cv[i], sv[i]);
    rhi[i] = rot_hi(lo[i], hi[i], cv[i], sv[i]);
  }
  uint32_t w_lo, w_hi;
  float mn, sc;
  encode8(rlo, rhi, gl, valid, w_lo, w_hi, mn, sc);
  if (valid) {
    *reinterpret_cast<uint32_t*>(a.out.k_codes + dst) = w_lo;
    *reinterpret_cast<uint32_t*>(a.out.k_codes + dst + half) = w_hi;
    if (lane_in == 0) *reinterpret_cast<float2*>(a.out.k_stats + (drow * hkv + h) * 2) = make_float2(mn, sc);
  }
  if constexpr (DEV) {
    // KVBoost page, section 4.6.2, Algorithm 2 at one layer: 1 - mean over
    // heads of cos(stored key, probe key); the stored key decodes as
    // min + code * scale, a head's cosine 0 when either norm is 0
    const BatchArgs& B = a.B;
    bool ctx = valid && drow < B.cu_T[B.n_req];
    int64_t jdx = 0;
    if (ctx) {
      const int r = find_segment(B.cu_T, B.n_req, static_cast<int>(drow));
      const int64_t i = drow - B.cu_T[r];
      ctx = i < B.n_ctx[r];
      jdx = B.cu_N[r] + i;
    }
    float dot = 0.f, nx = 0.f, ny = 0.f;
    if (ctx && score_eligible(a.dev, jdx)) {
      const u32x2_t fl = *reinterpret_cast<const u32x2_t*>(a.k_fresh + dst);
      const u32x2_t fh = *reinterpret_cast<const u32x2_t*>(a.k_fresh + dst + half);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float yl = __uint_as_float((i & 1) ? (fl[i >> 1] & 0xffff0000u) : (fl[i >> 1] << 16));
        const float yh = __uint_as_float((i & 1) ? (fh[i >> 1] & 0xffff0000u) : (fh[i >> 1] << 16));
        const float xl = fmaf(static_cast<float>((w_lo >> (8 * i)) & 0xffu), sc, mn);
        const float xh = fmaf(static_cast<float>((w_hi >> (8 * i)) & 0xffu), sc, mn);
        dot = fmaf(xl, yl, fmaf(xh, yh, dot));
        nx = fmaf(xl, xl, fmaf(xh, xh, nx));
        ny = fmaf(yl, yl, fmaf(yh, yh, ny));
      }
    }
    dot = group_sum(dot, gl);
    nx = group_sum(nx, gl);
    ny = group_sum(ny, gl);
    const float den = sqrtf(nx) * sqrtf(ny);
    float cs = (lane_in == 0 && den > 0.f) ? dot / den : 0.f;
    const int rl = hkv * gl;                       // lanes of one row
    cs = group_sum(cs, rl);
    if ((static_cast<int>(threadIdx.x) & (rl - 1)) == 0 && ctx)
      store_score(a.dev, jdx, 1.f - cs / static_cast<float>(hkv));
  }
  // values: 8-bit KIVI rows are copied, dense ones encoded
  if constexpr (KB == 8) {
    if (valid) {
      *reinterpret_cast<uint32_t*>(a.out.v_codes + dst) = *reinterpret_cast<const uint32_t*>(a.v_codes + src);
      *reinterpret_cast<uint32_t*>(a.out.v_codes + dst + half) =
          *reinterpret_cast<const uint32_t*>(a.v_codes + src + half);
      if (lane_in == 0)
        *reinterpret_cast<float2*>(a.out.v_stats + (drow * hkv + h) * 2) =
            make_float2(a.v_min[srow * hkv + h], a.v_scale[srow * hkv + h]);
    }
  } else {
    float vlo[4] = {0.f, 0.f, 0.f, 0.f}, vhi[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      const u32x2_t wl = *reinterpret_cast<const u32x2_t*>(a.pool_v + src);
      const u32x2_t wh = *reinterpret_cast<const u32x2_t*>(a.pool_v + src + half);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        vlo[2 * i] = __uint_as_float(wl[i] << 16);
        vlo[2 * i + 1] = __uint_as_float(wl[i] & 0xffff0000u);
        vhi[2 * i] = __uint_as_float(wh[i] << 16);
        vhi[2 * i + 1] = __uint_as_float(wh[i] & 0xffff0000u);
      }
    }
    encode8(vlo, vhi, gl, valid, w_lo, w_hi, mn, sc);
    if (valid) {
      *reinterpret_cast<uint32_t*>(a.out.v_codes + dst) = w_lo;
      *reinterpret_cast<uint32_t*>(a.out.v_codes + dst + half) = w_hi;
      if (lane_in == 0) *reinterpret_cast<float2*>(a.out.v_stats + (drow * hkv + h) * 2) = make_float2(mn, sc);
    }
  }
}

// Lanes of one fused row in rerotate_q8_kernel when the fused deviation
// score supports the shape (a power of two dividing 64, rows not straddling
// workgroups), else 0.
int rerotate_q8_deviation_lanes(int hkv, int d) {
  if (d % 32 != 0 || d < 32) return 0;
  const int gl = d / 8, rl = hkv * gl, ipb = kQ8RotWaves * kWave / gl;
  return (rl <= kWave && (rl & (rl - 1)) == 0 && ipb % hkv == 0) ? rl : 0;
}

hipError_t launch_rerotate_q8(const kvf_layer_desc& L, const kvf_chunk* chunks, int n_chunks,
                              int max_len, const void* pk, const void* pv, const kvf_kivi* q,
                              int64_t pool_rows, const float* rc, const float* rs, int rope_n,
                              const kvf_q8_cache& fused, hipStream_t st, const RotDeviation* dev) {
  RotQ8Args a{};
  a.chunks = chunks;
  a.pool_k = static_cast<const bf16_t*>(pk);
  a.pool_v = static_cast<const bf16_t*>(pv);
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
  a.out = fused;
  a.hkv = L.n_kv_heads;
  a.d = L.head_dim;
  const int ipb = kQ8RotWaves * kWave / (L.head_dim / 8);    // items per workgroup
  const int64_t gy = (static_cast<int64_t>(max_len) * L.n_kv_heads + ipb - 1) / ipb;
  if (gy > 65535) return hipErrorInvalidValue;
  const dim3 grid(n_chunks, static_cast<unsigned>(gy));
  if (dev) {
    if (rerotate_q8_deviation_lanes(a.hkv, a.d) == 0) return hipErrorInvalidValue;
    a.k_fresh = static_cast<const bf16_t*>(dev->k_fresh);
    a.dev = dev->out;
    a.B = dev->B;
    if (q)
      hipLaunchKernelGGL((rerotate_q8_kernel<8, true>), grid, dim3(64 * kQ8RotWaves), 0, st, a);
    else
      hipLaunchKernelGGL((rerotate_q8_kernel<0, true>), grid, dim3(64 * kQ8RotWaves), 0, st, a);
  } else if (q) {
    hipLaunchKernelGGL((rerotate_q8_kernel<8, false>), grid, dim3(64 * kQ8RotWaves), 0, st, a);
  } else {
    hipLaunchKernelGGL((rerotate_q8_kernel<0, false>), grid, dim3(64 * kQ8RotWaves), 0, st, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// offline KIVI encoder (not on the fused-layer path)
// ---------------------------------------------------------------------------
// keys: one thread per (pool chunk, head, code byte) - one channel for
// b = 8, the channel pair (2i, 2i+1) for b = 4; two passes over the chunk
template <int BITS>
__global__ void __launch_bounds__(256) kivi_keys_kernel(const bf16_t* __restrict__ pk,
                                                        const int32_t* __restrict__ pool_cu,
                                                        int n_pool, int64_t pool_rows, int hkv,
                                                        int d, uint8_t* __restrict__ codes,
                                                        float* __restrict__ kmin,
                                                        float* __restrict__ kscale) {
  constexpr int CPB = 8 / BITS;                            // channels per code byte
  const int c = blockIdx.y;
  const int byte = blockIdx.x * blockDim.x + threadIdx.x;  // code byte within a row
  const int row = hkv * d;
  const int row_bytes = row / CPB;
  if (c >= n_pool || byte >= row_bytes) return;
  const int a = pool_cu[c], b = pool_cu[c + 1];
  if (a < 0 || b < a || b > pool_rows) return;
  const int ch0 = byte * CPB;                              // head * d + channel
  float mn[CPB], mx[CPB], sc[CPB], inv[CPB];
#pragma unroll
  for (int q = 0; q < CPB; ++q) {
    mn[q] = INFINITY;
    mx[q] = -INFINITY;
  }
  for (int t = a; t < b; ++t)
#pragma unroll
    for (int q = 0; q < CPB; ++q) {
      const float x = bf16_to_f32(pk[static_cast<int64_t>(t) * row + ch0 + q]);
      mn[q] = fminf(mn[q], x);
      mx[q] = fmaxf(mx[q], x);
    }
#pragma unroll
  for (int q = 0; q < CPB; ++q) {
    if (b > a) {
      kivi_stats<BITS>(mn[q], mx[q], sc[q], inv[q]);
    } else {
      mn[q] = 0.f;
      sc[q] = inv[q] = 0.f;
    }
    kmin[static_cast<int64_t>(c) * row + ch0 + q] = mn[q];
    kscale[static_cast<int64_t>(c) * row + ch0 + q] = sc[q];
  }
  for (int t = a; t < b; ++t) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < CPB; ++q) {
      const float x = bf16_to_f32(pk[static_cast<int64_t>(t) * row + ch0 + q]);
      v |= kivi_code<BITS>(x, mn[q], inv[q]) << (BITS * q);
    }
    codes[static_cast<int64_t>(t) * row_bytes + byte] = static_cast<uint8_t>(v);
  }
}

// values: one wave per (row, head); a lane writes whole code bytes
template <int BITS>
__global__ void __launch_bounds__(256) kivi_values_kernel(const bf16_t* __restrict__ pv,
                                                          int64_t n_groups, int d,
                                                          uint8_t* __restrict__ codes,
                                                          float* __restrict__ vmin,
                                                          float* __restrict__ vscale) {
  constexpr int CPB = 8 / BITS;
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
  float sc, inv;
  kivi_stats<BITS>(mn, mx, sc, inv);
  if (lane == 0) {
    vmin[g] = mn;
    vscale[g] = sc;
  }
  const int gb = d / CPB;                                  // code bytes per group
  for (int k = lane; k < gb; k += kWave) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < CPB; ++q)
      v |= kivi_code<BITS>(bf16_to_f32(src[k * CPB + q]), mn, inv) << (BITS * q);
    codes[g * gb + k] = static_cast<uint8_t>(v);
  }
}

template <int BITS>
static hipError_t kivi_encode_bits(const kvf_layer_desc& L, const void* pk, const void* pv,
                                   const int32_t* pool_cu, int n_pool, int64_t pool_rows,
                                   const kvf_kivi& out, hipStream_t st) {
  const int hkv = L.n_kv_heads, d = L.head_dim;
  const int row_bytes = hkv * d * BITS / 8;
  hipLaunchKernelGGL(kivi_keys_kernel<BITS>, dim3(ceil_div(row_bytes, 256), n_pool), dim3(256), 0,
                     st, static_cast<const bf16_t*>(pk), pool_cu, n_pool, pool_rows, hkv, d,
                     const_cast<uint8_t*>(out.k_codes), const_cast<float*>(out.k_min),
                     const_cast<float*>(out.k_scale));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t groups = pool_rows * hkv;
  const int64_t blocks = (groups * kWave + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kivi_values_kernel<BITS>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     st, static_cast<const bf16_t*>(pv), groups, d,
                     const_cast<uint8_t*>(out.v_codes), const_cast<float*>(out.v_min),
                     const_cast<float*>(out.v_scale));
  return hipGetLastError();
}

hipError_t launch_kivi_encode(const kvf_layer_desc& L, const void* pk, const void* pv,
                              const int32_t* pool_cu, int n_pool, int64_t pool_rows, int max_len,
                              const kvf_kivi& out, hipStream_t st) {
  (void)max_len;
  if (n_pool > 65535) return hipErrorInvalidValue;
  return out.bits == 4 ? kivi_encode_bits<4>(L, pk, pv, pool_cu, n_pool, pool_rows, out, st)
                       : kivi_encode_bits<8>(L, pk, pv, pool_cu, n_pool, pool_rows, out, st);
}

}  // namespace kvf
