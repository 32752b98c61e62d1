// Token sampling and speculative-sampling acceptance on the GPU (gfx950).
//
// The Butter architecture notes (GPU sampling diagram) run sampling as a
// final kernel after the lm_head, so a decode loop reads back 4 bytes per
// token; oxinfer 0.0.5 docs ("Speculative decoding") accept sampled drafts
// with the standard speculative-sampling rule.  What is computed per logit
// row x (vocabulary V):
//   z = x / T (T = 0: greedy, the lowest index of the maximum);
//   top-k: keep z >= the k-th largest z (ties with it kept);
//   weights w = exp(z - max z) over the kept tokens;
//   top-p: the cut is the weight at which the mass of the heaviest tokens
//   first reaches p of the kept total; keep every token at or above it;
//   draw with u in [0, 1): the smallest index (index order) whose cumulative
//   kept weight exceeds u times the kept total.
//
// One workgroup per row.  The k-th largest value and the top-p cut are found
// by radix selection over the order-preserving 32-bit key of z, 8 bits per
// pass, from the top: a pass histograms the keys that share the prefix found
// so far (counts for top-k, weights for top-p), in one LDS histogram per
// wave, and the bin where the running count / weight from the top reaches
// the target extends the prefix.  Weights are summed as 64-bit fixed point
// (2^40 per unit), so every sum and every decision is independent of the
// order the threads add in: the same logits give the same token on every run.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int ST = 1024;       // threads per workgroup
constexpr int SW = ST / 64;    // waves
constexpr double FX = 1099511627776.0;  // 2^40: fixed-point unit of one weight (w <= 1)
typedef unsigned long long u64;

// Order-preserving key of a float (larger float, larger key; -0 as +0).
DPK_DEV uint32_t okey(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One row's sampling distribution: every token with key(z) >= cut has weight
// round(2^40 exp(z - zmax)), the others 0; total = the sum of the weights.
// greedy >= 0: T == 0, all mass on that index.
struct Dist {
  float zmax;
  uint32_t cut;
  int greedy;
  u64 total;
};

struct Lds {
  u64 hist[SW][256];   // per-wave histograms (counts use the low word)
  u64 sum[256];
  float fred[SW];
  int ired[SW];
  u64 ured[SW];
  Dist d;
  uint32_t sel_bin;
  u64 sel_need, sel_above;
  int result;
};

DPK_DEV float zval(const float* x, int i, float T) { return x[i] / T; }

DPK_DEV u64 weight_of(float z, const Dist& d) {
  if (okey(z) < d.cut) return 0ull;
  return (u64)rint((double)expf(z - d.zmax) * FX);
}

DPK_DEV u64 wave_sum_u64(u64 v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    v += ((u64)hi << 32) | lo;
  }
  return v;
}

DPK_DEV u64 block_sum_u64(u64 v, Lds& s) {
  v = wave_sum_u64(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.ured[w] = v;
  __syncthreads();
  u64 t = 0;
  for (int i = 0; i < SW; ++i) t += s.ured[i];
  return t;
}

// Radix-select one 8-bit digit: histogram (count or weight) of the keys that
// match prefix under mask, then find, from the top bin down, the bin where
// the running total reaches need.  Returns with s.sel_bin / s.sel_need (need
// left inside the bin) / s.sel_above (total above the bin) set.
template <bool MASS>
DPK_DEV void select_digit(const float* x, int V, float T, const Dist& d, uint32_t prefix, uint32_t mask, int shift,
                          u64 need, Lds& s) {
  const int tid = threadIdx.x, w = tid >> 6;
  for (int i = tid; i < SW * 256; i += ST) (&s.hist[0][0])[i] = 0ull;
  __syncthreads();
  for (int i = tid; i < V; i += ST) {
    const float z = zval(x, i, T);
    const uint32_t k = okey(z);
    if ((k & mask) == prefix && k >= d.cut) {
      const int b = (k >> shift) & 255;
      if (MASS)
        atomicAdd(&s.hist[w][b], weight_of(z, d));
      else
        atomicAdd((unsigned*)&s.hist[w][b], 1u);
    }
  }
  __syncthreads();
  for (int b = tid; b < 256; b += ST) {
    u64 t = 0;
    for (int ww = 0; ww < SW; ++ww) t += MASS ? s.hist[ww][b] : (u64)(*(unsigned*)&s.hist[ww][b]);
    s.sum[b] = t;
  }
  __syncthreads();
  if (tid == 0) {
    u64 above = 0;
    int b = 255;
    for (; b > 0; --b) {
      if (above + s.sum[b] >= need) break;
      above += s.sum[b];
    }
    s.sel_bin = (uint32_t)b;
    s.sel_need = need - above;
    s.sel_above = above;
  }
  __syncthreads();
}

// The distribution of row x (all threads return the same Dist).
DPK_DEV Dist row_dist(const float* x, int V, float T, int top_k, float top_p, Lds& s) {
  const int tid = threadIdx.x;
  Dist d{0.f, 0u, -1, 0ull};
  if (T == 0.f) {  // greedy: lowest index of the maximum
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = tid; i < V; i += ST) {
      const float v = x[i];
      if (v > bv) { bv = v; bi = i; }  // i grows: the first maximum seen is the lowest index
    }
    wave_argmax(bv, bi);
    __syncthreads();
    if ((tid & 63) == 0) { s.fred[tid >> 6] = bv; s.ired[tid >> 6] = bi; }
    __syncthreads();
    if (tid == 0) {
      float v = s.fred[0];
      int ix = s.ired[0];
      for (int w = 1; w < SW; ++w)
        if (s.fred[w] > v || (s.fred[w] == v && s.ired[w] < ix)) { v = s.fred[w]; ix = s.ired[w]; }
      s.d = Dist{0.f, 0u, ix, (u64)FX};
    }
    __syncthreads();
    return s.d;
  }
  float m = -INFINITY;
  for (int i = tid; i < V; i += ST) m = fmaxf(m, zval(x, i, T));
  m = wave_max(m);
  __syncthreads();
  if ((tid & 63) == 0) s.fred[tid >> 6] = m;
  __syncthreads();
  m = s.fred[0];
  for (int w = 1; w < SW; ++w) m = fmaxf(m, s.fred[w]);
  d.zmax = m;
  // top-k: the key of the k-th largest z
  if (top_k > 0 && top_k < V) {
    uint32_t prefix = 0, mask = 0;
    u64 need = (u64)top_k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      select_digit<false>(x, V, T, d, prefix, mask, shift, need, s);
      prefix |= s.sel_bin << shift;
      mask |= 0xFFu << shift;
      need = s.sel_need;
    }
    d.cut = prefix;
  }
  // kept total, and top-p: the largest key whose weight at and above it
  // reaches ceil(p * total)
  if (top_p < 1.f) {
    uint32_t prefix = 0, mask = 0;
    u64 need = 0, above = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (shift == 24) {
        // the first pass histograms every kept key: its sum is the total
        select_digit<true>(x, V, T, d, 0u, 0u, 24, ~0ull, s);
        u64 tot = 0;
        for (int b = 0; b < 256; ++b) tot += s.sum[b];
        need = (u64)ceil((double)top_p * (double)tot);
        if (need < 1) need = 1;
        if (need > tot) need = tot;
        // redo the bin search with the real target (the histogram is in s.sum)
        if (tid == 0) {
          u64 ab = 0;
          int b = 255;
          for (; b > 0; --b) {
            if (ab + s.sum[b] >= need) break;
            ab += s.sum[b];
          }
          s.sel_bin = (uint32_t)b;
          s.sel_need = need - ab;
          s.sel_above = ab;
        }
        __syncthreads();
      } else {
        select_digit<true>(x, V, T, d, prefix, mask, shift, need, s);
      }
      above += s.sel_above;
      prefix |= s.sel_bin << shift;
      mask |= 0xFFu << shift;
      need = s.sel_need;
    }
    // total kept = weight strictly above the cut key + weight at it
    d.total = above + s.sum[prefix & 255];
    d.cut = prefix;
  } else {
    u64 t = 0;
    for (int i = tid; i < V; i += ST) t += weight_of(zval(x, i, T), d);
    d.total = block_sum_u64(t, s);
  }
  return d;
}

// Smallest index whose cumulative weight (index order) exceeds tgt, for
// weights given by wf(i); tgt < the sum of all weights.  Each wave owns one
// contiguous segment: segment sums, then the owning wave scans its segment
// 64 elements at a time.
template <typename WF>
DPK_DEV int draw_index(int V, u64 tgt, WF&& wf, Lds& s) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int seg = ((V + SW - 1) / SW + 63) / 64 * 64;
  const int b0 = w * seg, b1 = min(V, b0 + seg);
  u64 t = 0;
  for (int i = b0 + lane; i < b1; i += 64) t += wf(i);
  t = wave_sum_u64(t);
  __syncthreads();
  if (lane == 0) s.ured[w] = t;
  if (tid == 0) s.result = -1;
  __syncthreads();
  u64 off = 0;
  int owner = -1;
  for (int ww = 0; ww < SW; ++ww) {
    if (owner < 0 && off + s.ured[ww] > tgt) owner = ww;
    else if (owner < 0) off += s.ured[ww];
  }
  if (owner < 0) {  // tgt beyond the total (not reached for tgt < total): last token with weight
    owner = SW - 1;
  }
  if (w == owner) {
    u64 run = off;
    int found = -1;
    for (int base = b0; base < b1 && found < 0; base += 64) {
      const int i = base + lane;
      const u64 v = i < b1 ? wf(i) : 0ull;
      // inclusive scan over the wave
      u64 inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t lo = __shfl_up((uint32_t)inc, o, 64), hi = __shfl_up((uint32_t)(inc >> 32), o, 64);
        if (lane >= o) inc += ((u64)hi << 32) | lo;
      }
      const bool hit = run + inc > tgt && v > 0;
      const u64 ball = __ballot(hit);
      if (ball) {
        found = base + __ffsll((long long)ball) - 1;
      } else {
        const uint32_t lo = __shfl((uint32_t)inc, 63, 64), hi = __shfl((uint32_t)(inc >> 32), 63, 64);
        run += ((u64)hi << 32) | lo;
      }
    }
    if (lane == 0) s.result = found >= 0 ? found : b1 - 1;
  }
  __syncthreads();
  return s.result;
}

DPK_DEV int sample_row(const float* x, int V, const Dist& d, float T, float u, Lds& s) {
  if (d.greedy >= 0) return d.greedy;
  u64 tgt = (u64)floor((double)u * (double)d.total);
  if (tgt >= d.total) tgt = d.total - 1;
  return draw_index(V, tgt, [&](int i) { return weight_of(zval(x, i, T), d); }, s);
}

// Probability of token t under a row's distribution (double).
DPK_DEV double prob_of(const float* x, int t, const Dist& d, float T) {
  if (d.greedy >= 0) return t == d.greedy ? 1.0 : 0.0;
  return (double)weight_of(zval(x, t, T), d) / (double)d.total;
}

__global__ __launch_bounds__(ST) void sample_kernel(const float* logits, long long ld, int V, float T, int top_k,
                                                    float top_p, const float* u, int* out) {
  __shared__ Lds s;
  const float* x = logits + (size_t)blockIdx.x * ld;
  const Dist d = row_dist(x, V, T, top_k, top_p, s);
  const int tok = sample_row(x, V, d, T, u[blockIdx.x], s);
  if (threadIdx.x == 0) out[blockIdx.x] = tok;
}

// Workgroup r < K + 1: target row r; K + 1 + i: draft row i.  Writes each
// row's distribution to ws.
__global__ __launch_bounds__(ST) void spec_dist_kernel(const float* target, const float* draft, long long ld, int V,
                                                       int K, float T, int top_k, float top_p, Dist* ws) {
  __shared__ Lds s;
  const int r = blockIdx.x;
  const float* x = r <= K ? target + (size_t)r * ld : draft + (size_t)(r - K - 1) * ld;
  const Dist d = row_dist(x, V, T, top_k, top_p, s);
  if (threadIdx.x == 0) ws[r] = d;
}

// Sequential acceptance of the K drafts, then the residual or bonus draw.
// out[0] = accepted count m, out[1] = the next token.
__global__ __launch_bounds__(ST) void spec_accept_kernel(const float* target, const float* draft, long long ld, int V,
                                                         int K, float T, const int* drafts, const float* r,
                                                         const float* u, const Dist* ws, int* out) {
  __shared__ Lds s;
  __shared__ int stop;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int m = 0;
    for (; m < K; ++m) {
      const int t = drafts[m];
      if (t < 0 || t >= V) break;  // an id outside the vocabulary is rejected (never read)
      const double p = prob_of(target + (size_t)m * ld, t, ws[m], T);
      const double q = prob_of(draft + (size_t)m * ld, t, ws[K + 1 + m], T);
      if (!((double)r[m] * q < p)) break;
    }
    stop = m;
  }
  __syncthreads();
  const int m = stop;
  int tok;
  if (m == K) {
    tok = sample_row(target + (size_t)K * ld, V, ws[K], T, u[K], s);
  } else {
    // residual max(0, p - q) in 2^50 fixed point of probability; if it is
    // zero everywhere (p == q) the draw is from p itself
    const float* xp = target + (size_t)m * ld;
    const float* xq = draft + (size_t)m * ld;
    const Dist dp = ws[m], dq = ws[K + 1 + m];
    const double FR = 1125899906842624.0;  // 2^50
    auto res = [&](int i) -> u64 {
      const double d = prob_of(xp, i, dp, T) - prob_of(xq, i, dq, T);
      return d > 0.0 ? (u64)rint(d * FR) : 0ull;
    };
    u64 t = 0;
    for (int i = tid; i < V; i += ST) t += res(i);
    const u64 tot = block_sum_u64(t, s);
    if (tot > 0) {
      u64 tgt = (u64)floor((double)u[m] * (double)tot);
      if (tgt >= tot) tgt = tot - 1;
      tok = draw_index(V, tgt, res, s);
    } else {
      tok = sample_row(xp, V, dp, T, u[m], s);
    }
  }
  if (tid == 0) {
    out[0] = m;
    out[1] = tok;
  }
}

// Workspace of the allocation-free acceptance entry point: the per-row
// distribution records of one call with up to SPEC_NOALLOC_MAX_K drafts.  One
// copy per GPU, shared by every call on that GPU (calls that overlap on one
// GPU race on it); each call writes every record it reads, so nothing needs
// clearing between calls.
constexpr int SPEC_NOALLOC_MAX_K = 16;
constexpr size_t SPEC_NOALLOC_BYTES = 4096;
static_assert((2 * SPEC_NOALLOC_MAX_K + 1) * sizeof(Dist) <= SPEC_NOALLOC_BYTES, "records fit the scratch array");
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_BYTES];

}  // namespace

size_t spec_dist_bytes(int K) { return (size_t)(2 * K + 1) * sizeof(Dist); }

int spec_noalloc_max_k() { return SPEC_NOALLOC_MAX_K; }

// Device address of `scratch` on the current device.  The array's name is a
// host-side stand-in in host code; its device address comes from the runtime,
// looked up once per device (with that device current) and kept.
hipError_t spec_noalloc_scratch(void** ptr) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* addr[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_sample(const float* logits, long long ld, int rows, int V, float T, int top_k, float top_p,
                         const float* u, int* out, hipStream_t stream) {
  if (rows < 1 || V < 1 || ld < V) return hipErrorInvalidValue;
  launch(sample_kernel, dim3(rows), dim3(ST), 0, stream, logits, ld, V, T, top_k, top_p, u, out);
  return hipGetLastError();
}

hipError_t launch_spec_accept(const float* target, const float* draft, long long ld, int V, int K, float T,
                              int top_k, float top_p, const int* drafts, const float* r, const float* u, void* ws,
                              int* out, hipStream_t stream) {
  if (K < 1 || V < 1 || ld < V) return hipErrorInvalidValue;
  launch(spec_dist_kernel, dim3(2 * K + 1), dim3(ST), 0, stream, target, draft, ld, V, K, T, top_k, top_p,
         (Dist*)ws);
  launch(spec_accept_kernel, dim3(1), dim3(ST), 0, stream, target, draft, ld, V, K, T, drafts, r, u,
         (const Dist*)ws, out);
  return hipGetLastError();
}

}  // namespace dpk
