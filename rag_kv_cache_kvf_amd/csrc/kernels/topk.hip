// S3: per-request top-k selection of context positions.
//
// QCFuse page, section 3.2.1, Eq. 11: P = TopK(I(t), floor(rho N)).  The order
// is larger score first, ties to the lower position (-0 == +0, NaN below
// every number); P is written ascending, followed (optionally) by the
// request's query rows so the caller gets the full recompute row list.
//
// One 1024-thread workgroup per request.  Scores map to order-preserving
// uint32 keys; an MSB-first 8-bit radix select (four LDS histogram passes)
// finds the k-th largest key tau and how many keys equal to tau are still
// needed.  A block-wide scan over per-thread contiguous segments then keeps
// every key above tau plus the first needed ties in index order and writes
// them in ascending order - no sort, and the result is exact.
#include "../kvf_common.h"

namespace kvf {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkCache = 36864;   // keys cached in LDS (144 KB)

struct TopkArgs {
  BatchArgs b;
  int k[KVF_MAX_REQ];
  int cu_k[KVF_MAX_REQ + 1];
  int cu_m[KVF_MAX_REQ + 1];
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;   // NaN below everything
  if (u == 0x80000000u) u = 0u;                     // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive block scan of one int per thread; also returns the block total
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) s_wave[w] = incl;
  __syncthreads();
  if (w == 0) {
    int x = lane < kTopkWaves ? s_wave[lane] : 0;
    int xi = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(xi, o, kWave);
      if (lane >= o) xi += t;
    }
    if (lane < kTopkWaves) s_wave[lane] = xi - x;      // exclusive wave offsets
    if (lane == kTopkWaves - 1) s_wave[kTopkWaves] = xi;
  }
  __syncthreads();
  const int res = s_wave[w] + incl - v;
  *total = s_wave[kTopkWaves];
  __syncthreads();
  return res;
}

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(TopkArgs a, const float* __restrict__ scores,
                                                            int32_t* __restrict__ out_idx,
                                                            int32_t* __restrict__ out_rows,
                                                            int32_t* __restrict__ out_pos) {
  // kCopies interleaved copies of the 256-bin histogram: lane l adds into
  // copy l % kCopies, and the stride kCopies + 1 puts the copies of one bin
  // in distinct LDS banks, so a wave whose keys share a bin (scores of one
  // request mostly share their top bits) costs a few conflict cycles instead
  // of 64 serialised atomics on one word.
  constexpr int kCopies = 8;
  __shared__ uint32_t hist[256 * (kCopies + 1)];
  __shared__ uint32_t s_sel[2];
  __shared__ int s_wave[kTopkWaves + 1];
  // the request's order keys, read from global memory once when they fit
  __shared__ uint32_t s_keys[kTopkCache];
  const int r = blockIdx.x;
  const int N = a.b.n_ctx[r];
  const int k = a.k[r];
  const int T = a.b.cu_T[r + 1] - a.b.cu_T[r];
  const int U = T - N;
  const float* sc = scores + a.b.cu_N[r];
  const int tid = threadIdx.x;
  const bool cached = N <= kTopkCache;
  if (cached && k > 0 && k < N)
    for (int i = tid; i < N; i += kTopkThreads) s_keys[i] = order_key(sc[i]);
  auto key_at = [&](int i) __attribute__((always_inline)) {
    return cached ? s_keys[i] : order_key(sc[i]);
  };

  uint32_t tau = 0u;        // keys > tau are taken; `need` keys == tau in index order
  int need = 0;
  if (k > 0 && k < N) {
    uint32_t prefix = 0u, mask = 0u;
    int krem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256 * (kCopies + 1); i += kTopkThreads) hist[i] = 0u;
      __syncthreads();
      const uint32_t copy = tid % kCopies;
      for (int i = tid; i < N; i += kTopkThreads) {
        const uint32_t key = key_at(i);
        if ((key & mask) == prefix) atomicAdd(&hist[((key >> shift) & 255u) * (kCopies + 1) + copy], 1u);
      }
      __syncthreads();
      // fold the copies into copy 0 of each bin
      for (int b = tid; b < 256; b += kTopkThreads) {
        uint32_t t = 0u;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) t += hist[b * (kCopies + 1) + c];
        hist[b * (kCopies + 1)] = t;
      }
      __syncthreads();
      if (tid < kWave) {
        // lane l owns bins 255-4l .. 252-4l (descending)
        const int b0 = 255 - 4 * tid;
        uint32_t c4[4];
        uint32_t sum4 = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c4[j] = hist[(b0 - j) * (kCopies + 1)];
          sum4 += c4[j];
        }
        uint32_t incl = sum4;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t t = __shfl_up(incl, o, kWave);
          if (tid >= o) incl += t;
        }
        const uint32_t excl = incl - sum4;
        if (excl < static_cast<uint32_t>(krem) && static_cast<uint32_t>(krem) <= incl) {
          uint32_t c = excl;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (c + c4[j] >= static_cast<uint32_t>(krem)) {
              s_sel[0] = prefix | (static_cast<uint32_t>(b0 - j) << shift);
              s_sel[1] = static_cast<uint32_t>(krem) - c;
              break;
            }
            c += c4[j];
          }
        }
      }
      __syncthreads();
      prefix = s_sel[0];
      krem = static_cast<int>(s_sel[1]);
      mask |= 255u << shift;
      __syncthreads();
    }
    tau = prefix;
    need = krem;
  }

  // compaction over contiguous per-thread segments
  const int seg = ceil_div(N, kTopkThreads);
  const int s0 = min(N, tid * seg), s1 = min(N, s0 + seg);
  int n_gt = 0, n_eq = 0;
  if (k == N) {
    n_gt = s1 - s0;
  } else if (k > 0) {
    for (int i = s0; i < s1; ++i) {
      const uint32_t key = key_at(i);
      n_gt += key > tau;
      n_eq += key == tau;
    }
  }
  int tot;
  const int eq_base = block_exclusive_scan(n_eq, s_wave, &tot);
  const int take = max(0, min(n_eq, need - eq_base));
  const int out_base = block_exclusive_scan(n_gt + take, s_wave, &tot);

  int32_t* oi = out_idx ? out_idx + a.cu_k[r] : nullptr;
  int32_t* orow = out_rows ? out_rows + a.cu_m[r] : nullptr;
  int32_t* opos = out_pos ? out_pos + a.cu_m[r] : nullptr;
  const int row0 = a.b.cu_T[r];
  if (k > 0) {
    int o = out_base, eq_seen = 0;
    for (int i = s0; i < s1; ++i) {
      bool sel;
      if (k == N) {
        sel = true;
      } else {
        const uint32_t key = key_at(i);
        sel = key > tau;
        if (key == tau) {
          sel = eq_seen < take;
          ++eq_seen;
        }
      }
      if (sel) {
        if (oi) oi[o] = i;
        if (orow) {
          orow[o] = row0 + i;
          opos[o] = i;
        }
        ++o;
      }
    }
  }
  if (orow) {
    for (int u = tid; u < U; u += kTopkThreads) {
      orow[k + u] = row0 + N + u;
      opos[k + u] = N + u;
    }
  }
}

hipError_t launch_topk(const float* scores, const BatchArgs& B, const int32_t* k_host,
                       int32_t* out_idx, int32_t* out_rows, int32_t* out_pos, hipStream_t st) {
  TopkArgs a{};
  a.b = B;
  for (int r = 0; r < B.n_req; ++r) {
    a.k[r] = k_host[r];
    a.cu_k[r + 1] = a.cu_k[r] + k_host[r];
    a.cu_m[r + 1] = a.cu_m[r] + k_host[r] + (B.cu_T[r + 1] - B.cu_T[r] - B.n_ctx[r]);
  }
  hipLaunchKernelGGL(topk_kernel, dim3(B.n_req), dim3(kTopkThreads), 0, st, a, scores, out_idx,
                     out_rows, out_pos);
  return hipGetLastError();
}

}  // namespace kvf
