// Static recompute positions: attention-sink tokens (KVBoost page, section
// 4.1), the first tokens of every stitched chunk (EPIC's boundary rule, QCFuse
// page, section 2.2.1) and the window of R tokens before every seam (KVBoost
// page, section 4.6.1, Algorithm 1).  The result is a byte mask over each
// request's context positions that the top-k selection takes as its forced
// set.
//
// One workgroup per request.  The mask is built in LDS, a window of
// kMaskWin positions at a time: clear (setting the sink), let every thread
// mark the ranges of the chunks it reads from the chunk table, then copy the
// window out with coalesced byte stores.  Marks of one position by several
// threads all store 1, so they need no atomics.
#include "../kvf_common.h"

namespace kvf {

constexpr int kMaskThreads = 256;
constexpr int kMaskWin = 16384;

struct StaticArgs {
  BatchArgs b;
  int sink;
  int boundary;
  int seam;
};

__global__ void __launch_bounds__(kMaskThreads) static_mask_kernel(StaticArgs a,
                                                                   const kvf_chunk* __restrict__ chunks,
                                                                   int n_chunks,
                                                                   uint8_t* __restrict__ mask) {
  __shared__ uint8_t win[kMaskWin];
  const int r = blockIdx.x;
  const int N = a.b.n_ctx[r];
  const int64_t row0 = a.b.cu_T[r];
  uint8_t* out = mask + a.b.cu_N[r];
  for (int w0 = 0; w0 < N; w0 += kMaskWin) {
    const int wl = min(kMaskWin, N - w0);
    for (int i = threadIdx.x; i < wl; i += kMaskThreads) win[i] = (w0 + i < a.sink) ? 1 : 0;
    __syncthreads();
    // [lo, hi) intersected with this window
    auto mark = [&](int64_t lo, int64_t hi) __attribute__((always_inline)) {
      const int l = static_cast<int>(max<int64_t>(lo, w0));
      const int h = static_cast<int>(min<int64_t>(hi, w0 + wl));
      for (int t = l; t < h; ++t) win[t - w0] = 1;
    };
    for (int c = threadIdx.x; c < n_chunks; c += kMaskThreads) {
      const int64_t p = static_cast<int64_t>(chunks[c].dst_row) - row0;
      if (p < 0 || p >= N) continue;
      mark(p, p + a.boundary);
      if (p > 0) mark(p - a.seam, p);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < wl; i += kMaskThreads) out[w0 + i] = win[i];
    __syncthreads();
  }
}

hipError_t launch_static_mask(const BatchArgs& B, const kvf_chunk* chunks, int n_chunks,
                              const kvf_static_rules& rules, uint8_t* mask, hipStream_t st) {
  StaticArgs a{};
  a.b = B;
  a.sink = rules.sink;
  a.boundary = rules.boundary;
  a.seam = rules.seam;
  hipLaunchKernelGGL(static_mask_kernel, dim3(B.n_req), dim3(kMaskThreads), 0, st, a, chunks,
                     n_chunks, mask);
  return hipGetLastError();
}

// The same marks on the host, counted per request.
void static_counts_host(const BatchArgs& B, const kvf_chunk* chunks, int n_chunks,
                        const kvf_static_rules& rules, int32_t* counts) {
  for (int r = 0; r < B.n_req; ++r) {
    const int N = B.n_ctx[r];
    std::vector<uint8_t> m(static_cast<size_t>(N), 0);
    auto mark = [&](int64_t lo, int64_t hi) {
      for (int64_t t = std::max<int64_t>(lo, 0); t < std::min<int64_t>(hi, N); ++t) m[t] = 1;
    };
    mark(0, rules.sink);
    for (int c = 0; c < n_chunks; ++c) {
      const int64_t p = static_cast<int64_t>(chunks[c].dst_row) - B.cu_T[r];
      if (p < 0 || p >= N) continue;
      mark(p, p + rules.boundary);
      if (p > 0) mark(p - rules.seam, p);
    }
    int32_t n = 0;
    for (uint8_t v : m) n += v;
    counts[r] = n;
  }
}

}  // namespace kvf
