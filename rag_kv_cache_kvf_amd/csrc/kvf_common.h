// Shared device/host definitions of libkvfuse (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "kvfuse.h"

namespace kvf {

constexpr int kWave = 64;
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kCUs = 256;         // MI355X: 32 compute units per XCD

using bf16_t = uint16_t;          // storage form of bf16 values

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// element traits: 8-wide loads/stores in fp32 registers
// ---------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<float> {
  static constexpr kvf_dtype kDtype = KVF_F32;
  __device__ __forceinline__ static void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store8(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

template <> struct Elem<bf16_t> {
  static constexpr kvf_dtype kDtype = KVF_BF16;
  __device__ __forceinline__ static void load8(const bf16_t* p, float (&v)[8]) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store8(bf16_t* p, const float (&v)[8]) {
    u32x4_t a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4_t*>(p) = a;
  }
  __device__ __forceinline__ static float load1(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store1(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// ---------------------------------------------------------------------------
// wave reductions (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// sum over aligned groups of `width` lanes (width a power of two <= 64)
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// min and max over aligned groups of `width` lanes (width a power of two <= 64)
__device__ __forceinline__ void group_minmax(float& mn, float& mx, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
}

// ---------------------------------------------------------------------------
// KIVI-style affine codes (KVBoost page, section 4.5, Eq. 7): fp32, in this
// order: range = max - min, scale = range / levels, inv = levels / range,
// code = (x - min) * inv rounded half to even and clamped to [0, levels];
// range 0 gives scale 0 and codes 0.  levels = 2^BITS - 1.
// ---------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ uint32_t kivi_code(float x, float mn, float inv) {
  constexpr float kTop = static_cast<float>((1 << BITS) - 1);
  const float t = (x - mn) * inv;
  return static_cast<uint32_t>(fminf(fmaxf(rintf(t), 0.f), kTop));
}

template <int BITS>
__device__ __forceinline__ void kivi_stats(float mn, float mx, float& sc, float& inv) {
  constexpr float kTop = static_cast<float>((1 << BITS) - 1);
  const float rng = mx - mn;
  sc = rng > 0.f ? rng / kTop : 0.f;
  inv = rng > 0.f ? kTop / rng : 0.f;
}

// ---------------------------------------------------------------------------
// hand-off between workgroups
// ---------------------------------------------------------------------------
// "The last workgroup to arrive combines": every workgroup stores its partial
// results with device-scope coherence (the sc1 cache policy: the store is
// written through to the level shared by all XCDs instead of staying in its
// own XCD's L2), then waits for its own stores to be acknowledged
// (s_waitcnt vmcnt(0): on gfx9-family parts vmcnt counts outstanding vector
// stores as well as loads, and a store is acknowledged once it has reached
// the coherence level its cache policy names), then the workgroup barrier
// orders that wait before one thread's counter bump.  The last arrival sees
// the count of every other workgroup, so every other workgroup's stores had
// completed before it bumped; it reads them with device-scope loads (which
// do not hit a stale line in its own L2).  This needs neither a release
// fence (an L2 write-back of the whole cache on this part) nor an acquire
// fence (an L2 invalidate), which evict the K/V tiles that other workgroups
// on the same XCD are streaming.
__device__ __forceinline__ void put_dev(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same coherence for 16-byte accesses: buffer loads/stores with the
// device-scope cache policy (sc1), through a descriptor over the hand-off
// buffer (byte offsets below 4 GiB).
constexpr int kDeviceScope = 16;                  // cache-policy bits: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t handoff_rsrc(void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                           0x00020000);
}
// Byte offset = voff (per lane) + soff (wave-uniform, a scalar register).
__device__ __forceinline__ void put_dev4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, voff, soff, kDeviceScope);
}
__device__ __forceinline__ f32x4_t get_dev4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kDeviceScope));
}
// 8- and 4-byte forms (plain loads and stores to the compiler, so a batch of
// them is issued back to back; relaxed atomics would be issued one at a
// time).
__device__ __forceinline__ void put_dev2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float x,
                                         float y) {
  const u32x2_t v = {__float_as_uint(x), __float_as_uint(y)};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, kDeviceScope);
}
__device__ __forceinline__ float2 get_dev2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kDeviceScope);
  return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
}
__device__ __forceinline__ void put_dev1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, kDeviceScope);
}
__device__ __forceinline__ float get_dev1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kDeviceScope));
}
// Every wave: wait until this wave's vector stores have been acknowledged,
// then the workgroup barrier.  (A plain __syncthreads() waits only for LDS
// traffic on this part, not for global stores.)  The memory clobber keeps
// the compiler from moving any store past the wait.
__device__ __forceinline__ void stores_done_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}
// All threads: true in the workgroup that arrived last of n at *cnt, which
// that workgroup sets back to zero for the next call.  Call it after the
// workgroup's device-scope partial stores.
__device__ __forceinline__ bool arrive_last(int* cnt, int n, int* s_flag) {
  stores_done_barrier();                          // every wave's stores have completed
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == n - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// ---------------------------------------------------------------------------
// batch metadata passed by value in kernel arguments
// ---------------------------------------------------------------------------
struct BatchArgs {
  int n_req;
  int cu_T[KVF_MAX_REQ + 1];   // row offsets of each request (x, fused cache)
  int n_ctx[KVF_MAX_REQ];      // context tokens N_r
  int cu_N[KVF_MAX_REQ + 1];   // offsets of each request's scores
  int cu_U[KVF_MAX_REQ + 1];   // offsets of each request's query rows (q_u)
};

// index of the request whose [cu[r], cu[r+1]) holds i (cu non-decreasing)
__device__ __forceinline__ int find_segment(const int* cu, int n, int i) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Where a score kernel writes.  A position whose eligibility byte is 0 gets
// NaN (ranked below every score by the selection); with `acc` the score is
// added to the value already there (scores summed over layers).
struct ScoreOut {
  float* scores;                // [sum N]
  const uint8_t* elig;          // [sum N] or nullptr (every position eligible)
  int acc;
};
__device__ __forceinline__ bool score_eligible(const ScoreOut& o, int64_t j) {
  return o.elig == nullptr || o.elig[j] != 0;
}
__device__ __forceinline__ void store_score(const ScoreOut& o, int64_t j, float v) {
  if (!score_eligible(o, j)) {
    o.scores[j] = __builtin_nanf("");
    return;
  }
  o.scores[j] = o.acc ? o.scores[j] + v : v;
}

}  // namespace kvf

// ---------------------------------------------------------------------------
// host-side launchers implemented in the kernel files
// ---------------------------------------------------------------------------
namespace kvf {
hipError_t launch_rope_table(double base, int d, int n_pos, float* c, float* s, hipStream_t st);
// The deviation score a re-positioning pass computes on the side
// (kvf_rerotate_deviation): k_fresh rows indexed like the fused cache.
struct RotDeviation {
  const void* k_fresh;
  ScoreOut out;
  BatchArgs B;
};
// rotation units per fused row if the fused deviation score supports the
// shape, else 0
int rerotate_deviation_lanes(int hkv, int d);
hipError_t launch_rerotate(const kvf_layer_desc& L, const kvf_chunk* chunks, int n_chunks,
                           int max_len, const void* pk, const void* pv, const kvf_kivi* q,
                           int64_t pool_rows, const float* rc, const float* rs, int rope_n,
                           void* fk, void* fv, int64_t fused_rows, int k_only, hipStream_t st,
                           const RotDeviation* dev = nullptr);
// int8-resident fused cache (kvf_q8_cache)
// rows' lanes in the int8-resident pass if its fused deviation score supports
// the shape, else 0
int rerotate_q8_deviation_lanes(int hkv, int d);
hipError_t launch_rerotate_q8(const kvf_layer_desc& L, const kvf_chunk* chunks, int n_chunks,
                              int max_len, const void* pk, const void* pv, const kvf_kivi* q,
                              int64_t pool_rows, const float* rc, const float* rs, int rope_n,
                              const kvf_q8_cache& fused, hipStream_t st,
                              const RotDeviation* dev = nullptr);
hipError_t launch_scatter_q8(const kvf_layer_desc& L, const void* ks, const int32_t* ksr,
                             int64_t ks_rows, const void* vs, const int32_t* vsr, int64_t vs_rows,
                             const int32_t* dst, int M, const kvf_q8_cache& fused, hipStream_t st);
hipError_t launch_deviation_q8(const kvf_layer_desc& L, const BatchArgs& B, const kvf_q8_cache& c,
                               const void* kf, const ScoreOut& out, hipStream_t st);
hipError_t launch_key_norm_q8(const kvf_layer_desc& L, const BatchArgs& B, const kvf_q8_cache& c,
                              const ScoreOut& out, hipStream_t st);
hipError_t launch_attention_q8(const kvf_layer_desc& L, const BatchArgs& B, const void* q,
                               const int32_t* q_pos, const int32_t* cu_q, const kvf_q8_cache& c,
                               float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                               hipStream_t st);
hipError_t launch_kivi_encode(const kvf_layer_desc& L, const void* pk, const void* pv,
                              const int32_t* pool_cu, int n_pool, int64_t pool_rows,
                              int max_len, const kvf_kivi& out, hipStream_t st);
hipError_t launch_deviation(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                            const void* kf, const ScoreOut& out, hipStream_t st);
// keys-only re-positioning fused into the attention-mass pass
// (kvf_rerotate_score_attn_mass)
struct MassRotate {
  const kvf_chunk* chunks;
  int n_chunks;
  int max_len;
  const void* pool_k;            // per-chunk keys (may be the fused cache: in place)
  int64_t pool_rows;
  const float* rope_cos;
  const float* rope_sin;
  int rope_n;
  int64_t fused_rows;
};
hipError_t launch_attn_mass(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                            const void* q_u, int n_last_q, const ScoreOut& out, void* ws,
                            size_t ws_bytes, hipStream_t st, const MassRotate* rot = nullptr);
size_t attn_mass_workspace(const kvf_layer_desc& L, const BatchArgs& B, int n_last_q);
hipError_t launch_attn_mass_noalloc(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                                    const void* q_u, int n_last_q, const ScoreOut& out,
                                    hipStream_t st);
// 128-key context tiles of a batch; the attention-mass call takes at most 16384
int64_t attn_mass_key_tiles(const BatchArgs& B);
hipError_t launch_key_norm(const kvf_layer_desc& L, const BatchArgs& B, const void* fk,
                           const ScoreOut& out, hipStream_t st);
hipError_t launch_topk(const float* scores, const uint8_t* forced, const BatchArgs& B,
                       const int32_t* k_host, int32_t* out_idx, int32_t* out_rows,
                       int32_t* out_pos, uint8_t* out_mask, hipStream_t st);
hipError_t launch_topk_segmented(const float* scores, const uint8_t* forced, const BatchArgs& B,
                                 const kvf_segment* segs, int n_segs, const int32_t* k_host,
                                 int32_t* out_idx, int32_t* out_rows, int32_t* out_pos,
                                 hipStream_t st);
hipError_t launch_static_mask(const BatchArgs& B, const kvf_chunk* chunks, int n_chunks,
                              const kvf_static_rules& rules, uint8_t* mask, hipStream_t st);
void static_counts_host(const BatchArgs& B, const kvf_chunk* chunks, int n_chunks,
                        const kvf_static_rules& rules, int32_t* counts);
hipError_t launch_recompute(const kvf_layer_desc& L, const void* x, int64_t x_rows,
                            const int32_t* row_src, const int32_t* row_pos, int M,
                            const void* w, uint32_t mask, const float* rc, const float* rs,
                            int rope_n, void* q, void* k, void* v, const int32_t* kv_row,
                            int64_t kv_rows, void* ws, size_t ws_bytes, hipStream_t st);
size_t recompute_workspace(const kvf_layer_desc& L, int M, uint32_t mask);
hipError_t launch_scatter(const kvf_layer_desc& L, const void* ks, const int32_t* ksr,
                          int64_t ks_rows, const void* vs, const int32_t* vsr, int64_t vs_rows,
                          const int32_t* dst, int M, void* fk, void* fv, int64_t fused_rows,
                          hipStream_t st);
hipError_t launch_attention(const kvf_layer_desc& L, const BatchArgs& B, const void* q,
                            const int32_t* q_pos, const int32_t* cu_q_host, const void* fk,
                            const void* fv, float sm_scale, void* out, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t st);
size_t attention_workspace(const kvf_layer_desc& L, const BatchArgs& B, const int32_t* cu_q_host);
}  // namespace kvf
