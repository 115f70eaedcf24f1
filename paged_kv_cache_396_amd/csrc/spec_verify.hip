// Verification of drafted tokens by rejection sampling (speculative decoding).
//
// zihan-zhang.net vLLM study, 4.1.1: a drafter proposes k tokens from its
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
// Two kernels.  The vocabulary is cut into 256-entry segments.  The first
// kernel spreads every request's segments over many workgroups (16 segments
// each, so a batch fills the chip) and stores each segment's weight sum in
// the caller's workspace.  The second takes one workgroup per request: it
// scans the segment sums for the segment that holds T and re-reads that
// segment alone to find the token.  Every workgroup decides acceptance
// itself (k scalar reads) rather than waiting for another kernel.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kSvThreads = 256;
constexpr int kSvWaves = kSvThreads / kWave;
constexpr int kSvSeg = 4 * kWave;        // vocabulary entries per segment
constexpr int kSvSegsPerWave = 4;
constexpr int kSvSegsPerGroup = kSvWaves * kSvSegsPerWave;

struct SpecVerifyParams {
  const float* target;       // [B][k+1][V]
  const float* draft;        // [B][k][V] or null (one-hot drafts)
  const int32_t* tokens;     // [B][k]
  const float* uniforms;     // [B][k+1]
  int32_t* out_tokens;       // [B][k+1]
  int32_t* num_out;          // [B]
  uint64_t* seg_ws;          // [B][nseg] segment weight sums
  int k;
  int vocab;
  int nseg;
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

// The distribution request b draws its last token from, once the first
// rejected position i (k if none) is known.
struct SvRow {
  const float* p;  // p_i
  const float* q;  // q_i, or null
  int onehot;      // q_i one-hot at this token (drafts without distribution), or -1
  int V;
  __device__ uint64_t weight(int j, bool use_q) const {
    if (j >= V) return 0;
    float r = p[j];
    if (use_q) {
      if (q) r = r - q[j];
      else if (j == onehot) r = r - 1.f;
    }
    return sv_weight(r);
  }
};

// First rejected candidate of request b (k if all are kept), for every
// thread of the workgroup.
__device__ inline int sv_first_rejection(const SpecVerifyParams& p, int b, int* s_first) {
  const int k = p.k, V = p.vocab, tid = threadIdx.x;
  const float* tp = p.target + (int64_t)b * (k + 1) * V;
  const float* dp = p.draft ? p.draft + (int64_t)b * k * V : nullptr;
  if (tid == 0) *s_first = k;
  __syncthreads();
  if (tid < k) {
    const int x = p.tokens[(int64_t)b * k + tid];
    bool keep = false;
    if (x >= 0 && x < V) {
      const double pv = tp[(int64_t)tid * V + x];
      const double qv = dp ? (double)dp[(int64_t)tid * V + x] : 1.0;
      keep = (double)p.uniforms[(int64_t)b * (k + 1) + tid] * qv <= pv;
    }
    if (!keep) atomicMin(s_first, tid);
  }
  __syncthreads();
  return *s_first;
}

__device__ inline SvRow sv_row(const SpecVerifyParams& p, int b, int i) {
  const int k = p.k, V = p.vocab;
  SvRow r;
  r.p = p.target + ((int64_t)b * (k + 1) + i) * V;
  const int x = i < k ? p.tokens[(int64_t)b * k + i] : -1;
  const bool x_ok = x >= 0 && x < V;
  r.q = (i < k && p.draft && x_ok) ? p.draft + ((int64_t)b * k + i) * V : nullptr;
  r.onehot = (i < k && !p.draft && x_ok) ? x : -1;
  r.V = V;
  return r;
}

// Weight sum of segment s: lane l adds entries s*256 + 64e + l, e = 0..3
// (each load instruction reads 256 contiguous bytes).
__device__ inline uint64_t sv_segment_sum(const SvRow& row, int s, bool use_q, int lane) {
  uint64_t acc = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc += row.weight(s * kSvSeg + e * kWave + lane, use_q);
  return wave_sum_u64(acc);
}

// ---- kernel 1: segment sums of (p_i - q_i)_+ or p_k, spread over the chip
__global__ __launch_bounds__(kSvThreads) void spec_segments_kernel(SpecVerifyParams p) {
  __shared__ int s_first;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int i = sv_first_rejection(p, b, &s_first);
  const SvRow row = sv_row(p, b, i);
  const bool use_q = i < p.k;
  const int s0 = blockIdx.x * kSvSegsPerGroup + wv * kSvSegsPerWave;
  // all loads of the wave's segments first, then the sums
  float pv[kSvSegsPerWave][4], qv[kSvSegsPerWave][4];
#pragma unroll
  for (int t = 0; t < kSvSegsPerWave; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = (s0 + t) * kSvSeg + e * kWave + lane;
      const bool in = j < row.V;
      pv[t][e] = in ? row.p[j] : 0.f;
      qv[t][e] = (in && use_q && row.q) ? row.q[j] : 0.f;
    }
#pragma unroll
  for (int t = 0; t < kSvSegsPerWave; ++t) {
    const int s = s0 + t;
    if (s >= p.nseg) break;  // uniform over the wave
    uint64_t acc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = s * kSvSeg + e * kWave + lane;
      float r = pv[t][e];
      if (use_q) {
        if (row.q) r = r - qv[t][e];
        else if (j == row.onehot) r = r - 1.f;
      }
      acc += j < row.V ? sv_weight(r) : 0;
    }
    acc = wave_sum_u64(acc);
    if (lane == 0) p.seg_ws[(int64_t)b * p.nseg + s] = acc;
  }
}

// ---- kernel 2: one workgroup per request finds the token and writes the
// outputs.  A residual without weight is redone here from p_i alone.
__global__ __launch_bounds__(kSvThreads) void spec_select_kernel(SpecVerifyParams p) {
  extern __shared__ uint64_t seg_sum[];  // fallback pass only
  __shared__ uint64_t chunk_sum[kSvThreads];
  __shared__ int s_first;
  __shared__ int s_token;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int k = p.k;
  const int nseg = p.nseg;
  const int i = sv_first_rejection(p, b, &s_first);
  const SvRow row = sv_row(p, b, i);
  const float ui = p.uniforms[(int64_t)b * (k + 1) + k];
  const uint64_t* ws = p.seg_ws + (int64_t)b * nseg;

  int token = -1;
  for (int pass = 0; pass < 2; ++pass) {
    const bool use_q = pass == 0 && i < k;
    // pass 0 reads the first kernel's sums; pass 1 (p_i alone) makes its own
    const uint64_t* sums = ws;
    if (pass == 1) {
      for (int s = wv; s < nseg; s += kSvWaves) {
        const uint64_t v = sv_segment_sum(row, s, false, lane);
        if (lane == 0) seg_sum[s] = v;
      }
      __syncthreads();
      sums = seg_sum;
    }
    // thread t owns segments [t * C, t * C + C)
    const int C = (nseg + kSvThreads - 1) / kSvThreads;
    {
      uint64_t acc = 0;
      for (int s = tid * C; s < min(nseg, tid * C + C); ++s) acc += sums[s];
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
        // first lane whose running sum passes T, then its chunk
        const uint64_t hit = __ballot(incl > T);
        const int L = __ffsll((unsigned long long)hit) - 1;
        uint64_t base = __shfl(incl - lsum, L, kWave);
        int chunk = -1;
        for (int e = 0; e < 4; ++e) {
          const uint64_t ce = __shfl(c4[e], L, kWave);
          if (chunk < 0 && base + ce > T) chunk = L * 4 + e;
          else if (chunk < 0) base += ce;
        }
        // the chunk's segments, 64 at a time
        const int cend = min(nseg, chunk * C + C);
        int seg = -1;
        for (int s0 = chunk * C; seg < 0 && s0 < cend; s0 += kWave) {
          const int s = s0 + lane;
          const uint64_t v = s < cend ? sums[s] : 0;
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
        // the segment's entries in order, 64 at a time
        for (int e = 0; tok < 0 && e < 4; ++e) {
          const int j = seg * kSvSeg + e * kWave + lane;
          const uint64_t v = row.weight(j, use_q);
          const uint64_t in3 = wave_scan_u64(v, lane) + base;
          const uint64_t h3 = __ballot(in3 > T);
          if (h3) tok = seg * kSvSeg + e * kWave + __ffsll((unsigned long long)h3) - 1;
          else base = __shfl(in3, kWave - 1, kWave);
        }
      }
      if (lane == 0) s_token = tok;
    }
    __syncthreads();
    token = s_token;
    if (token >= 0 || !(i < k)) break;  // uniform: an empty p_k has nothing to fall back to
    __syncthreads();                    // chunk_sum is rewritten by the second pass
  }

  // ---- outputs: kept drafts, the drawn token, -1 padding
  int32_t* out = p.out_tokens + (int64_t)b * (k + 1);
  const int32_t* toks = p.tokens + (int64_t)b * k;
  for (int t = tid; t <= k; t += kSvThreads) out[t] = t < i ? toks[t] : (t == i ? token : -1);
  if (tid == 0) p.num_out[b] = i + 1;
}

size_t spec_verify_workspace_bytes(int num_reqs, int vocab) {
  const int64_t nseg = ((int64_t)vocab + kSvSeg - 1) / kSvSeg;
  return (size_t)((int64_t)num_reqs * nseg * (int64_t)sizeof(uint64_t));
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
  p.seg_ws = (uint64_t*)a.workspace;
  p.k = a.k;
  p.vocab = a.vocab;
  p.nseg = (a.vocab + kSvSeg - 1) / kSvSeg;
  const int groups = (p.nseg + kSvSegsPerGroup - 1) / kSvSegsPerGroup;
  if (a.num_reqs > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(spec_segments_kernel, dim3((unsigned)groups, (unsigned)a.num_reqs),
                     dim3(kSvThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_select_kernel, dim3((unsigned)a.num_reqs), dim3(kSvThreads),
                     (size_t)p.nseg * sizeof(uint64_t), stream, p);
  return hipGetLastError();
}

}  // namespace pa
