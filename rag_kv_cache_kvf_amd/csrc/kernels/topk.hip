// S3: top-k selection of context positions, whole-request and per-segment.
//
// QCFuse page, section 3.2.1, Eq. 11: P = TopK(I(t), floor(rho N)).  The order
// is larger score first, ties to the lower position (-0 == +0, NaN below
// every number); P is written ascending, followed (optionally) by the
// request's query rows so the caller gets the full recompute row list.
// A forced mask (positions every selection keeps: attention-sink tokens,
// KVBoost page, section 4.1; seam windows, section 4.6.1; EPIC's boundary
// tokens, QCFuse page, section 2.2.1) ranks its positions above every score,
// so they take the budget first, lowest positions first when they overflow it.
// The segmented form runs one selection per segment - the per-chunk anchors
// A_i = TopK(G_i, ceil(r_a |c_i|)) of QCFuse, section 3.3.1, Eq. 14 - so no
// chunk can take another chunk's budget.
//
// One workgroup per selection.  Scores map to order-preserving uint32 keys;
// an MSB-first 8-bit radix select (four LDS histogram passes) finds the k-th
// largest key tau and how many keys equal to tau are still needed.  A
// block-wide scan over per-thread contiguous segments then keeps every key
// above tau plus the first needed ties in index order and writes them in
// ascending order - no sort, and the result is exact.
#include "../kvf_common.h"

namespace kvf {

constexpr int kTopkThreads = 1024;
constexpr int kTopkCache = 36864;     // keys cached in LDS (144 KB)
constexpr int kSegThreads = 256;
constexpr int kSegCache = 8192;       // 32 KB: several segment workgroups per CU
constexpr int kHistCopies = 8;
constexpr uint32_t kForcedKey = 0xffffffffu;   // above the key of +inf (0xff800000)

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
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  constexpr int kWaves = NT / kWave;
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
    int x = lane < kWaves ? s_wave[lane] : 0;
    int xi = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(xi, o, kWave);
      if (lane >= o) xi += t;
    }
    if (lane < kWaves) s_wave[lane] = xi - x;      // exclusive wave offsets
    if (lane == kWaves - 1) s_wave[kWaves] = xi;
  }
  __syncthreads();
  const int res = s_wave[w] + incl - v;
  *total = s_wave[kWaves];
  __syncthreads();
  return res;
}

// LDS of one selecting workgroup.  kHistCopies interleaved copies of the
// 256-bin histogram: lane l adds into copy l % kHistCopies, and the stride
// kHistCopies + 1 puts the copies of one bin in distinct LDS banks, so a wave
// whose keys share a bin (scores of one request mostly share their top bits)
// costs a few conflict cycles instead of 64 serialised atomics on one word.
template <int NT, int CACHE>
struct SelectLds {
  uint32_t hist[256 * (kHistCopies + 1)];
  uint32_t sel[2];
  int wave[NT / kWave + 1];
  uint32_t keys[CACHE];     // the selection's keys, read from HBM once when they fit
};

// LDS slot of key i: one pad word after every 32 keys.  The compaction reads
// contiguous per-thread segments (thread t reads key t * seg + j at step j);
// with seg = 32 (32768 keys, 1024 threads) every lane of a wave would hit
// the same bank without the pad, with it the stride is 33 words.
__device__ __forceinline__ int key_slot(int i) { return i + (i >> 5); }

// The k largest keys of positions [0, N) with ties to the lower position;
// emit(o, i) is called for the o-th chosen position i, o ascending with i.
// sc == nullptr ranks every unforced position equal (lowest positions win).
// mask (optional): mask[i] = 1 for chosen positions, 0 for the others.
template <int NT, int CACHE, typename Emit>
__device__ __forceinline__ void select_block(const float* __restrict__ sc,
                                             const uint8_t* __restrict__ forced, int N, int k,
                                             SelectLds<NT, CACHE>& s, uint8_t* __restrict__ mask,
                                             Emit emit) {
  const int tid = threadIdx.x;
  auto key_of = [&](int i) __attribute__((always_inline)) -> uint32_t {
    if (forced && forced[i]) return kForcedKey;
    return sc ? order_key(sc[i]) : 0u;
  };
  const bool cached = key_slot(N) <= CACHE;
  if (cached && k > 0 && k < N)
    for (int i = tid; i < N; i += NT) s.keys[key_slot(i)] = key_of(i);
  auto key_at = [&](int i) __attribute__((always_inline)) {
    return cached ? s.keys[key_slot(i)] : key_of(i);
  };

  uint32_t tau = 0u;        // keys > tau are taken; `need` keys == tau in index order
  int need = 0;
  if (k > 0 && k < N && !sc) {
    // two key values only (forced, 0): one counting pass instead of the radix
    int f = 0;
    for (int i = tid; i < N; i += NT) f += key_at(i) == kForcedKey;
    int n_forced;
    block_exclusive_scan<NT>(f, s.wave, &n_forced);
    tau = k <= n_forced ? kForcedKey : 0u;
    need = k <= n_forced ? k : k - n_forced;
  } else if (k > 0 && k < N) {
    uint32_t prefix = 0u, mask = 0u;
    int krem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256 * (kHistCopies + 1); i += NT) s.hist[i] = 0u;
      __syncthreads();
      const uint32_t copy = tid % kHistCopies;
      for (int i = tid; i < N; i += NT) {
        const uint32_t key = key_at(i);
        if ((key & mask) == prefix)
          atomicAdd(&s.hist[((key >> shift) & 255u) * (kHistCopies + 1) + copy], 1u);
      }
      __syncthreads();
      // fold the copies into copy 0 of each bin
      for (int b = tid; b < 256; b += NT) {
        uint32_t t = 0u;
#pragma unroll
        for (int c = 0; c < kHistCopies; ++c) t += s.hist[b * (kHistCopies + 1) + c];
        s.hist[b * (kHistCopies + 1)] = t;
      }
      __syncthreads();
      if (tid < kWave) {
        // lane l owns bins 255-4l .. 252-4l (descending)
        const int b0 = 255 - 4 * tid;
        uint32_t c4[4];
        uint32_t sum4 = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c4[j] = s.hist[(b0 - j) * (kHistCopies + 1)];
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
              s.sel[0] = prefix | (static_cast<uint32_t>(b0 - j) << shift);
              s.sel[1] = static_cast<uint32_t>(krem) - c;
              break;
            }
            c += c4[j];
          }
        }
      }
      __syncthreads();
      prefix = s.sel[0];
      krem = static_cast<int>(s.sel[1]);
      mask |= 255u << shift;
      __syncthreads();
    }
    tau = prefix;
    need = krem;
  }

  // compaction over contiguous per-thread segments
  const int seg = ceil_div(N, NT);
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
  const int eq_base = block_exclusive_scan<NT>(n_eq, s.wave, &tot);
  const int take = max(0, min(n_eq, need - eq_base));
  const int out_base = block_exclusive_scan<NT>(n_gt + take, s.wave, &tot);
  auto decide = [&](int i, int& eq_seen) __attribute__((always_inline)) {
    if (k == 0) return false;
    if (k == N) return true;
    const uint32_t key = key_at(i);
    if (key != tau) return key > tau;
    return eq_seen++ < take;
  };
  if (cached && seg <= 32) {
    // Decisions as a bit mask over the thread's segment, then the picks are
    // laid out in LDS (over the key cache, no longer read) and written out
    // in index order by consecutive threads: coalesced stores instead of
    // each lane writing its own run of up to 32 scattered words.
    uint32_t bits = 0u;
    int eq_seen = 0;
    for (int i = s0; i < s1; ++i)
      if (decide(i, eq_seen)) bits |= 1u << (i - s0);
    __syncthreads();                              // every key read is done
    uint32_t* picks = s.keys;                     // k <= N entries fit
    int o = out_base;
    for (uint32_t b = bits; b; b &= b - 1) picks[o++] = static_cast<uint32_t>(s0 + __builtin_ctz(b));
    if (mask) s.hist[tid] = bits;                 // the histogram is no longer read
    __syncthreads();
    for (int o2 = tid; o2 < k; o2 += NT) emit(o2, static_cast<int>(picks[o2]));
    if (mask)
      for (int i = tid; i < N; i += NT) {
        const int t = i / seg;
        mask[i] = static_cast<uint8_t>((s.hist[t] >> (i - t * seg)) & 1u);
      }
  } else if (k > 0 || mask) {
    int o = out_base, eq_seen = 0;
    for (int i = s0; i < s1; ++i) {
      const bool sel = decide(i, eq_seen);
      if (mask) mask[i] = sel ? 1 : 0;
      if (sel) emit(o++, i);
    }
  }
}

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(TopkArgs a, const float* __restrict__ scores,
                                                            const uint8_t* __restrict__ forced,
                                                            int32_t* __restrict__ out_idx,
                                                            int32_t* __restrict__ out_rows,
                                                            int32_t* __restrict__ out_pos,
                                                            uint8_t* __restrict__ out_mask) {
  __shared__ SelectLds<kTopkThreads, kTopkCache> lds;
  const int r = blockIdx.x;
  const int N = a.b.n_ctx[r];
  const int k = a.k[r];
  const int T = a.b.cu_T[r + 1] - a.b.cu_T[r];
  const int U = T - N;
  const int row0 = a.b.cu_T[r];
  int32_t* oi = out_idx ? out_idx + a.cu_k[r] : nullptr;
  int32_t* orow = out_rows ? out_rows + a.cu_m[r] : nullptr;
  int32_t* opos = out_pos ? out_pos + a.cu_m[r] : nullptr;
  select_block<kTopkThreads, kTopkCache>(
      scores ? scores + a.b.cu_N[r] : nullptr, forced ? forced + a.b.cu_N[r] : nullptr, N, k, lds,
      out_mask ? out_mask + a.b.cu_N[r] : nullptr, [&](int o, int i) __attribute__((always_inline)) {
        if (oi) oi[o] = i;
        if (orow) {
          orow[o] = row0 + i;
          opos[o] = i;
        }
      });
  if (orow) {
    for (int u = threadIdx.x; u < U; u += kTopkThreads) {
      orow[k + u] = row0 + N + u;
      opos[k + u] = N + u;
    }
  }
}

// Blocks [0, n_segs) select one segment each; block n_segs + r writes the
// query rows of request r behind its picks.  A segment that breaks its
// contract (request, range, k or output slots out of bounds) writes nothing.
__global__ void __launch_bounds__(kSegThreads) topk_segmented_kernel(
    TopkArgs a, const float* __restrict__ scores, const uint8_t* __restrict__ forced,
    const kvf_segment* __restrict__ segs, int n_segs, int32_t* __restrict__ out_idx,
    int32_t* __restrict__ out_rows, int32_t* __restrict__ out_pos) {
  __shared__ SelectLds<kSegThreads, kSegCache> lds;
  if (static_cast<int>(blockIdx.x) >= n_segs) {
    const int r = blockIdx.x - n_segs;
    if (!out_rows) return;
    const int N = a.b.n_ctx[r];
    const int U = a.b.cu_T[r + 1] - a.b.cu_T[r] - N;
    for (int u = threadIdx.x; u < U; u += kSegThreads) {
      out_rows[a.cu_m[r] + a.k[r] + u] = a.b.cu_T[r] + N + u;
      out_pos[a.cu_m[r] + a.k[r] + u] = N + u;
    }
    return;
  }
  const kvf_segment g = segs[blockIdx.x];
  const int r = g.req;
  if (r < 0 || r >= a.b.n_req) return;
  const int N = a.b.n_ctx[r];
  if (g.pos0 < 0 || g.len < 0 || g.pos0 > N - g.len || g.k < 0 || g.k > g.len ||
      g.out_off < 0 || g.out_off > a.k[r] - g.k)
    return;
  const int base = a.b.cu_N[r] + g.pos0;
  const int row0 = a.b.cu_T[r] + g.pos0;
  int32_t* oi = out_idx ? out_idx + a.cu_k[r] + g.out_off : nullptr;
  int32_t* orow = out_rows ? out_rows + a.cu_m[r] + g.out_off : nullptr;
  int32_t* opos = out_pos ? out_pos + a.cu_m[r] + g.out_off : nullptr;
  select_block<kSegThreads, kSegCache>(
      scores ? scores + base : nullptr, forced ? forced + base : nullptr, g.len, g.k, lds, nullptr,
      [&](int o, int i) __attribute__((always_inline)) {
        if (oi) oi[o] = g.pos0 + i;
        if (orow) {
          orow[o] = row0 + i;
          opos[o] = g.pos0 + i;
        }
      });
}

static TopkArgs topk_args(const BatchArgs& B, const int32_t* k_host) {
  TopkArgs a{};
  a.b = B;
  for (int r = 0; r < B.n_req; ++r) {
    a.k[r] = k_host[r];
    a.cu_k[r + 1] = a.cu_k[r] + k_host[r];
    a.cu_m[r + 1] = a.cu_m[r] + k_host[r] + (B.cu_T[r + 1] - B.cu_T[r] - B.n_ctx[r]);
  }
  return a;
}

hipError_t launch_topk(const float* scores, const uint8_t* forced, const BatchArgs& B,
                       const int32_t* k_host, int32_t* out_idx, int32_t* out_rows,
                       int32_t* out_pos, uint8_t* out_mask, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3(B.n_req), dim3(kTopkThreads), 0, st, topk_args(B, k_host),
                     scores, forced, out_idx, out_rows, out_pos, out_mask);
  return hipGetLastError();
}

hipError_t launch_topk_segmented(const float* scores, const uint8_t* forced, const BatchArgs& B,
                                 const kvf_segment* segs, int n_segs, const int32_t* k_host,
                                 int32_t* out_idx, int32_t* out_rows, int32_t* out_pos,
                                 hipStream_t st) {
  hipLaunchKernelGGL(topk_segmented_kernel, dim3(n_segs + B.n_req), dim3(kSegThreads), 0, st,
                     topk_args(B, k_host), scores, forced, segs, n_segs, out_idx, out_rows,
                     out_pos);
  return hipGetLastError();
}

}  // namespace kvf
