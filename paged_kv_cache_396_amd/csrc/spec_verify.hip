// Verification of drafted tokens by rejection sampling (speculative decoding).
//
// plumephp.com vLLM deep dive, 4.1.1: a drafter proposes k tokens from its
// distributions q_i; the target model's distributions p_0..p_k come from one
// forward pass over all k + 1 positions (its attention is pa_prefill_chunk
// with k + 1 query rows per request).  Candidate x_i is kept with
// probability min(1, p_i(x_i) / q_i(x_i)); the first rejection ends the
// round with a token drawn from the normalised (p_i - q_i)_+, and a round
// whose k candidates all survive adds a bonus token drawn from p_k.
//
// Randomness is an input (uniforms u_0..u_k per request).  Decisions are
// exact, so every implementation of the same rule picks the same tokens:
//  * keep x_i iff u_i * q_i(x_i) <= p_i(x_i), the product of two fp32 values
//    formed exactly in fp64 (with q one-hot when drafts carry no
//    distribution; a draft token outside the vocabulary is never kept);
//  * draw by inverse CDF over integer weights w_j = floor(max(r_j, 0) * 2^32)
//    with r_j = p_j - q_j in fp32 (NaN counts as 0): the token is the first j
//    whose running weight sum exceeds T = floor(u_k * W), W the total weight,
//    T held below W; integer sums do not depend on the order of summation.
//    An empty residual (W = 0) draws from p_i instead.
//
// One workgroup per request.  The vocabulary is cut into 256-entry segments:
// a first pass sums each segment's weights (one wave per segment, 4 entries
// per lane), a scan over the segment sums finds the segment holding T, and
// one wave re-reads that segment alone to find the token.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kSvThreads = 256;
constexpr int kSvWaves = kSvThreads / kWave;
constexpr int kSvSeg = 4 * kWave;  // vocabulary entries per segment

struct SpecVerifyParams {
  const float* target;       // [B][k+1][V]
  const float* draft;        // [B][k][V] or null (one-hot drafts)
  const int32_t* tokens;     // [B][k]
  const float* uniforms;     // [B][k+1]
  int32_t* out_tokens;       // [B][k+1]
  int32_t* num_out;          // [B]
  int k;
  int vocab;
};

__device__ inline uint64_t sv_weight(float r) {
  r = fminf(fmaxf(r, 0.f), 1048576.f);  // NaN -> 0; the clamp only guards the conversion
  return (uint64_t)(r * 4294967296.f);  // exact scaling by 2^32, truncation = floor
}

// T = floor(u * W) held inside [0, W - 1]; exact: u = m * 2^-sh with a 24-bit m.
__device__ inline uint64_t sv_threshold(float u, uint64_t W) {
  if (!(u > 0.f)) return 0;
  if (u >= 1.f) return W - 1;
  const uint32_t bits = __float_as_uint(u);
  const int e = (int)((bits >> 23) & 0xffu);
  uint64_t m = bits & 0x7fffffu;
  int sh = 149;
  if (e != 0) {
    m |= 0x800000u;
    sh = 150 - e;
  }
  const unsigned __int128 prod = (unsigned __int128)m * W;
  const uint64_t t = sh >= 128 ? 0 : (uint64_t)(prod >> sh);
  return t < W ? t : W - 1;
}

__device__ inline uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// inclusive prefix sum over the 64 lanes
__device__ inline uint64_t wave_scan_u64(uint64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint64_t n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

__global__ __launch_bounds__(kSvThreads) void spec_verify_kernel(SpecVerifyParams p) {
  extern __shared__ uint64_t seg_sum[];  // one per 256-entry segment
  __shared__ uint64_t chunk_sum[kSvThreads];
  __shared__ int s_first;
  __shared__ int s_token;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int k = p.k;
  const int V = p.vocab;
  const float* tp = p.target + (int64_t)b * (k + 1) * V;
  const float* dp = p.draft ? p.draft + (int64_t)b * k * V : nullptr;
  const int32_t* toks = p.tokens + (int64_t)b * k;
  const float* u = p.uniforms + (int64_t)b * (k + 1);

  // ---- acceptance of every candidate; the first rejection ends the round
  if (tid == 0) s_first = k;
  __syncthreads();
  if (tid < k) {
    const int x = toks[tid];
    bool keep = false;
    if (x >= 0 && x < V) {
      const double pv = tp[(int64_t)tid * V + x];
      const double qv = dp ? (double)dp[(int64_t)tid * V + x] : 1.0;
      keep = (double)u[tid] * qv <= pv;
    }
    if (!keep) atomicMin(&s_first, tid);
  }
  __syncthreads();
  const int i = s_first;

  // ---- the distribution the last token comes from: (p_i - q_i)_+ after a
  // rejection at i, p_k after k acceptances
  const float* prow = tp + (int64_t)i * V;
  const int xi = i < k ? toks[i] : -1;
  const bool x_ok = xi >= 0 && xi < V;
  const float* qrow = (i < k && dp && x_ok) ? dp + (int64_t)i * V : nullptr;
  const int onehot = (i < k && !dp && x_ok) ? xi : -1;  // q one-hot at the draft token
  const int nseg = (V + kSvSeg - 1) / kSvSeg;
  const float ui = u[k];

  int token = -1;
  for (int pass = 0; pass < 2 && token < 0; ++pass) {
    const bool use_q = pass == 0 && i < k;
    if (pass == 1 && !(i < k)) break;  // p_k had no weight: nothing to fall back to
    auto weight_at = [&](int j) -> uint64_t {
      if (j >= V) return 0;
      float r = prow[j];
      if (use_q) {
        if (qrow) r = r - qrow[j];
        else if (j == onehot) r = r - 1.f;
      }
      return sv_weight(r);
    };
    // segment sums, one wave per segment
    for (int s = wv; s < nseg; s += kSvWaves) {
      const int j0 = s * kSvSeg + lane * 4;
      uint64_t acc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += weight_at(j0 + e);
      acc = wave_sum_u64(acc);
      if (lane == 0) seg_sum[s] = acc;
    }
    __syncthreads();
    // thread t owns segments [t * C, t * C + C)
    const int C = (nseg + kSvThreads - 1) / kSvThreads;
    {
      uint64_t acc = 0;
      for (int s = tid * C; s < min(nseg, tid * C + C); ++s) acc += seg_sum[s];
      chunk_sum[tid] = acc;
    }
    __syncthreads();
    if (wv == 0) {
      // scan the 256 chunk sums: lane l holds chunks 4l .. 4l+3
      uint64_t c4[4], lsum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = chunk_sum[lane * 4 + e];
        lsum += c4[e];
      }
      const uint64_t incl = wave_scan_u64(lsum, lane);
      const uint64_t W = __shfl(incl, kWave - 1, kWave);
      int tok = -1;
      if (W > 0) {
        const uint64_t T = sv_threshold(ui, W);
        // first lane whose running sum passes T
        const uint64_t hit = __ballot(incl > T);
        const int L = __ffsll((unsigned long long)hit) - 1;
        uint64_t base = __shfl(incl - lsum, L, kWave);  // weight before lane L's chunks
        int chunk = -1;
        for (int e = 0; e < 4; ++e) {
          const uint64_t ce = __shfl(c4[e], L, kWave);
          if (chunk < 0 && base + ce > T) chunk = L * 4 + e;
          else if (chunk < 0) base += ce;
        }
        // segments of that chunk, at most 64 of them per pass over the lanes
        int seg = -1;
        for (int s0 = chunk * C; seg < 0 && s0 < min(nseg, chunk * C + C); s0 += kWave) {
          const int s = s0 + lane;
          const uint64_t v = s < min(nseg, chunk * C + C) ? seg_sum[s] : 0;
          const uint64_t in2 = wave_scan_u64(v, lane) + base;
          const uint64_t h2 = __ballot(in2 > T);
          if (h2) {
            const int L2 = __ffsll((unsigned long long)h2) - 1;
            seg = s0 + L2;
            base = __shfl(in2 - v, L2, kWave);
          } else {
            base = __shfl(in2, kWave - 1, kWave);
          }
        }
        // entries of that segment: lane l holds 4l .. 4l+3
        const int j0 = seg * kSvSeg + lane * 4;
        uint64_t w4[4], l4 = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w4[e] = weight_at(j0 + e);
          l4 += w4[e];
        }
        const uint64_t in3 = wave_scan_u64(l4, lane) + base;
        const uint64_t h3 = __ballot(in3 > T);
        const int L3 = __ffsll((unsigned long long)h3) - 1;
        if (lane == L3) {
          uint64_t run = in3 - l4;
          for (int e = 0; e < 4; ++e) {
            run += w4[e];
            if (run > T) {
              tok = j0 + e;
              break;
            }
          }
        }
        tok = __shfl(tok, L3, kWave);
      }
      if (lane == 0) s_token = tok;
    }
    __syncthreads();
    token = s_token;
    __syncthreads();  // seg_sum / chunk_sum are rewritten by a second pass
  }

  // ---- outputs: kept drafts, the drawn token, -1 padding
  int32_t* out = p.out_tokens + (int64_t)b * (k + 1);
  for (int t = tid; t <= k; t += kSvThreads) out[t] = t < i ? toks[t] : (t == i ? token : -1);
  if (tid == 0) p.num_out[b] = i + 1;
}

hipError_t launch_spec_verify(const SpecVerifyArgs& a, hipStream_t stream) {
  if (a.num_reqs == 0) return hipSuccess;
  SpecVerifyParams p;
  p.target = a.target_probs;
  p.draft = a.draft_probs;
  p.tokens = a.draft_tokens;
  p.uniforms = a.uniforms;
  p.out_tokens = a.out_tokens;
  p.num_out = a.num_out;
  p.k = a.k;
  p.vocab = a.vocab;
  const int nseg = (a.vocab + kSvSeg - 1) / kSvSeg;
  hipLaunchKernelGGL(spec_verify_kernel, dim3((unsigned)a.num_reqs), dim3(kSvThreads),
                     (size_t)nseg * sizeof(uint64_t), stream, p);
  return hipGetLastError();
}

}  // namespace pa
