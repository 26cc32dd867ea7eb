// S5 in-place K/V scatter into the fused cache (bf16 or int8-resident), S2
// key-deviation score and the key-norm ranking score (reading either cache).
//
// Scatter: QCFuse page, section 2.1.3, Eq. 7 - the fused cache takes the
// recomputed entry at every selected position and keeps the reused one
// elsewhere; entries are written back at the same positions.
// Deviation: KVBoost page, section 4.6.2, Algorithm 2 - delta_t = 1 minus the
// mean over heads of cos(K_t, K~_t), here for one layer and the key heads.
//
// Key norm: QCFuse page, section 3.3.1 - the Knorm rule ranks a chunk's
// positions by the norm of their cached keys (one norm over all kv heads).
//
// All three are HBM streams.  Scatter moves 16-byte vectors with a
// grid-stride loop over (row, vector); deviation and key norm give each
// context token one wave that reads the key rows with 16-byte loads and
// reduces with cross-lane shuffles.
#include "../kvf_common.h"

namespace kvf {

// ---------------------------------------------------------------------------
// S5: scatter
// ---------------------------------------------------------------------------
struct ScatterArgs {
  const uint8_t* k_src;
  const int32_t* k_src_row;
  int64_t k_src_rows;
  const uint8_t* v_src;
  const int32_t* v_src_row;
  int64_t v_src_rows;
  const int32_t* dst_row;
  int M;
  uint8_t* fused_k;
  uint8_t* fused_v;
  int64_t fused_rows;
  int row_vecs;          // 16-byte vectors per row
};

__global__ void __launch_bounds__(256) scatter_kernel(ScatterArgs a) {
  const int64_t total = static_cast<int64_t>(a.M) * a.row_vecs;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t row_bytes = static_cast<int64_t>(a.row_vecs) * 16;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += stride) {
    const int m = static_cast<int>(i / a.row_vecs);
    const int v = static_cast<int>(i - static_cast<int64_t>(m) * a.row_vecs);
    const int32_t dst = a.dst_row[m];
    if (dst < 0 || dst >= a.fused_rows) continue;
    if (a.k_src) {
      const int64_t s = a.k_src_row ? a.k_src_row[m] : m;
      if (s >= 0 && s < a.k_src_rows) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(a.k_src + s * row_bytes + v * 16);
        *reinterpret_cast<u32x4_t*>(a.fused_k + dst * row_bytes + v * 16) = x;
      }
    }
    if (a.v_src) {
      const int64_t s = a.v_src_row ? a.v_src_row[m] : m;
      if (s >= 0 && s < a.v_src_rows) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(a.v_src + s * row_bytes + v * 16);
        *reinterpret_cast<u32x4_t*>(a.fused_v + dst * row_bytes + v * 16) = x;
      }
    }
  }
}

hipError_t launch_scatter(const kvf_layer_desc& L, const void* ks, const int32_t* ksr,
                          int64_t ks_rows, const void* vs, const int32_t* vsr, int64_t vs_rows,
                          const int32_t* dst, int M, void* fk, void* fv, int64_t fused_rows,
                          hipStream_t st) {
  ScatterArgs a{};
  a.k_src = static_cast<const uint8_t*>(ks);
  a.k_src_row = ksr;
  a.k_src_rows = ks_rows;
  a.v_src = static_cast<const uint8_t*>(vs);
  a.v_src_row = vsr;
  a.v_src_rows = vs_rows;
  a.dst_row = dst;
  a.M = M;
  a.fused_k = static_cast<uint8_t*>(fk);
  a.fused_v = static_cast<uint8_t*>(fv);
  a.fused_rows = fused_rows;
  const int esz = L.dtype == KVF_BF16 ? 2 : 4;
  a.row_vecs = L.n_kv_heads * L.head_dim * esz / 16;
  const int64_t total = static_cast<int64_t>(M) * a.row_vecs;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 16);
  hipLaunchKernelGGL(scatter_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// S5 into an int8-resident fused cache: work items are (recomputed row, kv
// head, tensor), d/8 lanes each; a lane loads 8 consecutive bf16 values (16
// bytes), the item's min/max is reduced over its lanes, and the lane stores
// its 8 codes as one 8-byte word.
struct ScatterQ8Args {
  const bf16_t* k_src;
  const int32_t* k_src_row;
  int64_t k_src_rows;
  const bf16_t* v_src;
  const int32_t* v_src_row;
  int64_t v_src_rows;
  const int32_t* dst_row;
  int M;
  kvf_q8_cache out;
  int hkv;
  int d;
};

__global__ void __launch_bounds__(256) scatter_q8_kernel(ScatterQ8Args a) {
  const int gl = a.d >> 3;                         // lanes per item
  const int64_t item = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / gl;
  const int lane_in = threadIdx.x & (gl - 1);
  // item = (m * hkv + h) * 2 + tensor (0: K, 1: V)
  const int tensor = static_cast<int>(item & 1);
  const int64_t mh = item >> 1;
  const int64_t m = mh / a.hkv;
  const int h = static_cast<int>(mh - m * a.hkv);
  const bf16_t* src = tensor ? a.v_src : a.k_src;
  const int32_t* srow_map = tensor ? a.v_src_row : a.k_src_row;
  const int64_t src_rows = tensor ? a.v_src_rows : a.k_src_rows;
  bool valid = m < a.M && src != nullptr;
  int64_t dst = 0, s = 0;
  if (valid) {
    dst = a.dst_row[m];
    s = srow_map ? srow_map[m] : m;
    valid = dst >= 0 && dst < a.out.rows && s >= 0 && s < src_rows;
  }
  float x[8];
  float mn = INFINITY, mx = -INFINITY;
  if (valid) {
    Elem<bf16_t>::load8(src + (s * a.hkv + h) * a.d + 8 * lane_in, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
  }
  // every lane of the wave takes part in the reduction
  group_minmax(mn, mx, gl);
  if (!valid) return;
  float sc, inv;
  kivi_stats<8>(mn, mx, sc, inv);
  u32x2_t w = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i >> 2] |= kivi_code<8>(x[i], mn, inv) << (8 * (i & 3));
  uint8_t* codes = tensor ? a.out.v_codes : a.out.k_codes;
  float* stats = tensor ? a.out.v_stats : a.out.k_stats;
  *reinterpret_cast<u32x2_t*>(codes + (dst * a.hkv + h) * a.d + 8 * lane_in) = w;
  if (lane_in == 0) *reinterpret_cast<float2*>(stats + (dst * a.hkv + h) * 2) = make_float2(mn, sc);
}

hipError_t launch_scatter_q8(const kvf_layer_desc& L, const void* ks, const int32_t* ksr,
                             int64_t ks_rows, const void* vs, const int32_t* vsr, int64_t vs_rows,
                             const int32_t* dst, int M, const kvf_q8_cache& fused, hipStream_t st) {
  ScatterQ8Args a{};
  a.k_src = static_cast<const bf16_t*>(ks);
  a.k_src_row = ksr;
  a.k_src_rows = ks_rows;
  a.v_src = static_cast<const bf16_t*>(vs);
  a.v_src_row = vsr;
  a.v_src_rows = vs_rows;
  a.dst_row = dst;
  a.M = M;
  a.out = fused;
  a.hkv = L.n_kv_heads;
  a.d = L.head_dim;
  const int64_t threads = static_cast<int64_t>(M) * L.n_kv_heads * 2 * (L.head_dim / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scatter_q8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Eight consecutive key elements e0..e0+7 (one head) of fused row `row`,
// in fp32: bf16/fp32 caches as stored, int8-resident ones decoded.
template <typename T>
struct KeyRow {
  const T* k;
  __device__ __forceinline__ void load8(int64_t row, int row_elems, int e0, float (&x)[8]) const {
    Elem<T>::load8(k + row * row_elems + e0, x);
  }
};
template <>
struct KeyRow<uint8_t> {
  const uint8_t* k;
  const float* st;
  int d;
  __device__ __forceinline__ void load8(int64_t row, int row_elems, int e0, float (&x)[8]) const {
    const u32x2_t c = *reinterpret_cast<const u32x2_t*>(k + row * row_elems + e0);
    const int64_t g = row * (row_elems / d) + e0 / d;
    const float2 ms = *reinterpret_cast<const float2*>(st + 2 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      x[i] = fmaf(static_cast<float>((c[i >> 2] >> (8 * (i & 3))) & 0xffu), ms.y, ms.x);
  }
};

// ---------------------------------------------------------------------------
// S2: key deviation
// ---------------------------------------------------------------------------
template <typename T, typename KR>
__global__ void __launch_bounds__(256) deviation_kernel(BatchArgs B, KR fk,
                                                        const T* __restrict__ kf, int hkv, int d,
                                                        ScoreOut out) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int total = B.cu_N[B.n_req];
  if (wave >= total) return;
  if (!score_eligible(out, wave)) {             // the whole wave: one token
    if (lane == 0) store_score(out, wave, 0.f);
    return;
  }
  const int r = find_segment(B.cu_N, B.n_req, wave);
  const int64_t row = B.cu_T[r] + (wave - B.cu_N[r]);
  const int row_elems = hkv * d;
  const int lanes_per_head = d >> 3;           // 8 elements per lane
  const T* b = kf + row * row_elems;
  float cos_acc = 0.f;
  for (int e0 = lane * 8; e0 < row_elems; e0 += kWave * 8) {
    float x[8], y[8];
    fk.load8(row, row_elems, e0, x);
    Elem<T>::load8(b + e0, y);
    float dot = 0.f, nx = 0.f, ny = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dot = fmaf(x[i], y[i], dot);
      nx = fmaf(x[i], x[i], nx);
      ny = fmaf(y[i], y[i], ny);
    }
    dot = group_sum(dot, lanes_per_head);
    nx = group_sum(nx, lanes_per_head);
    ny = group_sum(ny, lanes_per_head);
    const float den = sqrtf(nx) * sqrtf(ny);
    if ((lane & (lanes_per_head - 1)) == 0 && den > 0.f) cos_acc += dot / den;
  }
  // lanes past the row end still take part in the shuffles above with zeros
  cos_acc = wave_sum(cos_acc);
  if (lane == 0) store_score(out, wave, 1.f - cos_acc / static_cast<float>(hkv));
}

// Narrow rows: a row of Hkv d <= 256 elements (8 per lane) fills
// LPT = Hkv d / 8 lanes (a power of two), and 64 / LPT tokens share a wave
// instead of leaving its other lanes idle (Hkv = 2, d = 128: two per wave).
template <typename T, typename KR, int LPT>
__global__ void __launch_bounds__(256) deviation_packed_kernel(BatchArgs B, KR fk,
                                                        const T* __restrict__ kf, int hkv, int d,
                                                        ScoreOut out) {
  constexpr int TPW = kWave / LPT;              // tokens per wave
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane & (LPT - 1);
  const int total = B.cu_N[B.n_req];
  if (static_cast<int64_t>(wave) * TPW >= total) return;     // the whole wave
  const int tok = wave * TPW + lane / LPT;
  // lanes of a token past the end or not eligible load nothing, but take
  // part in the shuffles (with zeros) like every other lane of the wave
  const bool live = tok < total && score_eligible(out, tok);
  int64_t row = 0;
  if (live) {
    const int r = find_segment(B.cu_N, B.n_req, tok);
    row = B.cu_T[r] + (tok - B.cu_N[r]);
  }
  const int row_elems = hkv * d;
  const int lanes_per_head = d >> 3;           // 8 elements per lane
  const T* b = kf + row * row_elems;
  float cos_acc = 0.f;
  for (int e0 = sub * 8; e0 < row_elems; e0 += LPT * 8) {
    float x[8], y[8];
    if (live) {
      fk.load8(row, row_elems, e0, x);
      Elem<T>::load8(b + e0, y);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = y[i] = 0.f;
    }
    float dot = 0.f, nx = 0.f, ny = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dot = fmaf(x[i], y[i], dot);
      nx = fmaf(x[i], x[i], nx);
      ny = fmaf(y[i], y[i], ny);
    }
    dot = group_sum(dot, lanes_per_head);
    nx = group_sum(nx, lanes_per_head);
    ny = group_sum(ny, lanes_per_head);
    const float den = sqrtf(nx) * sqrtf(ny);
    if ((sub & (lanes_per_head - 1)) == 0 && den > 0.f) cos_acc += dot / den;
  }
  // lanes past the row end still take part in the shuffles above with zeros
  cos_acc = group_sum(cos_acc, LPT);
  if (sub == 0 && tok < total) store_score(out, tok, live ? 1.f - cos_acc / static_cast<float>(hkv) : 0.f);
}

// Lanes per token for a row of `row_elems` elements (see deviation_packed_kernel).
static int deviation_lanes(int row_elems) {
  const int l = row_elems / 8;
  return (row_elems % 8 == 0 && l <= 32 && (l & (l - 1)) == 0 && l >= 8) ? l : kWave;
}

template <typename T, typename KR>
static void launch_deviation_lanes(const BatchArgs& B, KR fk, const T* kf, int hkv, int d,
                                   const ScoreOut& out, hipStream_t st) {
  const int total = B.cu_N[B.n_req];
  const int lpt = deviation_lanes(hkv * d);
  const int waves = ceil_div(total, kWave / lpt);
  const int blocks = ceil_div(waves, 256 / kWave);
  switch (lpt) {
    case 8:
      hipLaunchKernelGGL((deviation_packed_kernel<T, KR, 8>), dim3(blocks), dim3(256), 0, st, B, fk, kf, hkv, d, out);
      break;
    case 16:
      hipLaunchKernelGGL((deviation_packed_kernel<T, KR, 16>), dim3(blocks), dim3(256), 0, st, B, fk, kf, hkv, d,
                         out);
      break;
    case 32:
      hipLaunchKernelGGL((deviation_packed_kernel<T, KR, 32>), dim3(blocks), dim3(256), 0, st, B, fk, kf, hkv, d,
                         out);
      break;
    default:                                   // one wave per token
      hipLaunchKernelGGL((deviation_kernel<T, KR>), dim3(blocks), dim3(256), 0, st, B, fk, kf, hkv, d, out);
  }
}

hipError_t launch_deviation(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                            const void* kf, const ScoreOut& out, hipStream_t st) {
  if (B.cu_N[B.n_req] == 0) return hipGetLastError();
  if (L.dtype == KVF_BF16)
    launch_deviation_lanes<bf16_t>(B, KeyRow<bf16_t>{static_cast<const bf16_t*>(fk)},
                                   static_cast<const bf16_t*>(kf), L.n_kv_heads, L.head_dim, out, st);
  else
    launch_deviation_lanes<float>(B, KeyRow<float>{static_cast<const float*>(fk)},
                                  static_cast<const float*>(kf), L.n_kv_heads, L.head_dim, out, st);
  return hipGetLastError();
}

hipError_t launch_deviation_q8(const kvf_layer_desc& L, const BatchArgs& B, const kvf_q8_cache& c,
                               const void* kf, const ScoreOut& out, hipStream_t st) {
  if (B.cu_N[B.n_req] == 0) return hipGetLastError();
  launch_deviation_lanes<bf16_t>(B, KeyRow<uint8_t>{c.k_codes, c.k_stats, L.head_dim},
                                 static_cast<const bf16_t*>(kf), L.n_kv_heads, L.head_dim, out, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// key norm
// ---------------------------------------------------------------------------
template <typename KR>
__global__ void __launch_bounds__(256) key_norm_kernel(BatchArgs B, KR fk, int row_elems,
                                                       ScoreOut out) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int total = B.cu_N[B.n_req];
  if (wave >= total) return;
  if (!score_eligible(out, wave)) {
    if (lane == 0) store_score(out, wave, 0.f);
    return;
  }
  const int r = find_segment(B.cu_N, B.n_req, wave);
  const int64_t row = B.cu_T[r] + (wave - B.cu_N[r]);
  float ss = 0.f;
  for (int e0 = lane * 8; e0 < row_elems; e0 += kWave * 8) {
    float x[8];
    fk.load8(row, row_elems, e0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) store_score(out, wave, sqrtf(ss));
}

hipError_t launch_key_norm(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                           const ScoreOut& out, hipStream_t st) {
  const int total = B.cu_N[B.n_req];
  const int blocks = ceil_div(total, 256 / kWave);
  const int row_elems = L.n_kv_heads * L.head_dim;
  if (L.dtype == KVF_BF16)
    hipLaunchKernelGGL(key_norm_kernel<KeyRow<bf16_t>>, dim3(blocks), dim3(256), 0, st, B,
                       KeyRow<bf16_t>{static_cast<const bf16_t*>(fk)}, row_elems, out);
  else
    hipLaunchKernelGGL(key_norm_kernel<KeyRow<float>>, dim3(blocks), dim3(256), 0, st, B,
                       KeyRow<float>{static_cast<const float*>(fk)}, row_elems, out);
  return hipGetLastError();
}

hipError_t launch_key_norm_q8(const kvf_layer_desc& L, const BatchArgs& B, const kvf_q8_cache& c,
                              const ScoreOut& out, hipStream_t st) {
  const int total = B.cu_N[B.n_req];
  const int blocks = ceil_div(total, 256 / kWave);
  const int row_elems = L.n_kv_heads * L.head_dim;
  hipLaunchKernelGGL(key_norm_kernel<KeyRow<uint8_t>>, dim3(blocks), dim3(256), 0, st, B,
                     KeyRow<uint8_t>{c.k_codes, c.k_stats, L.head_dim}, row_elems, out);
  return hipGetLastError();
}

}  // namespace kvf
