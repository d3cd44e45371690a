// HBM-bound kernels: LSE merge, backward preprocess (delta), zigzag
// gather/scatter.
#include "common.h"

namespace cpattn {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack8(const void* p, bool bf16, float* out) {
  if (bf16) {
    const u32x4 raw = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(raw[i] << 16);
      out[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
  } else {
    const f32x4 a = ((const f32x4*)p)[0], b = ((const f32x4*)p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
  }
}

// ---------------------------------------------------------------------------
// LSE merge.  Ring Attention ("Scaling Video Training with Parallelism",
// section 2) produces one partial (out, lse) per key/value block; two partial
// results over disjoint key sets combine as the softmax over their union:
//   lse' = m + log(exp(lse - m) + exp(lse_p - m)),  m = max(lse, lse_p)
//   out' = exp(lse - lse') out + exp(lse_p - lse') out_p
// Rows are visited head-major (r = h*T + t) so LSE traffic is contiguous and
// every (t, h) row of `out` is one contiguous run of d floats.  Each thread
// owns 8 elements of a row; a row with lse_p = -inf is neither read nor
// written (exact pass-through).
// ---------------------------------------------------------------------------


template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 8;  // threads per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / TPR;
  const int c = (int)(gid - r * TPR);
  if (r >= (int64_t)a.heads * a.tokens) return;
  const int h = (int)(r / a.tokens);
  const int64_t t = r - (int64_t)h * a.tokens;
  const float lp = a.lsep[r];
  if (lp == -INFINITY) return;
  const float lo = a.lse[r];
  float* orow = a.out + (t * a.heads + h) * D + c * 8;
  const char* prow = (const char*)a.op + ((t * a.op_st + (int64_t)h * a.op_sh) + c * 8) * (BF16 ? 2 : 4);
  float p[8];
  unpack8(prow, BF16, p);
  float w_o, w_p, nl;
  if (lo == -INFINITY) {
    w_o = 0.f; w_p = 1.f; nl = lp;
  } else {
    const float m = fmaxf(lo, lp);
    const float eo = __expf(lo - m), ep = __expf(lp - m);
    const float s = eo + ep;
    nl = m + __logf(s);
    const float inv = 1.f / s;
    w_o = eo * inv;
    w_p = ep * inv;
  }
  f32x4 o0 = ((f32x4*)orow)[0], o1 = ((f32x4*)orow)[1];
  if (lo == -INFINITY) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { o0[i] = p[i]; o1[i] = p[4 + i]; }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o0[i] = w_o * o0[i] + w_p * p[i];
      o1[i] = w_o * o1[i] + w_p * p[4 + i];
    }
  }
  ((f32x4*)orow)[0] = o0;
  ((f32x4*)orow)[1] = o1;
  if (c == 0) a.lse[r] = nl;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.heads * a.tokens * (a.d / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (a.d == 128) {
    if (a.bf16) hipLaunchKernelGGL((merge_kernel<128, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((merge_kernel<128, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.bf16) hipLaunchKernelGGL((merge_kernel<64, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((merge_kernel<64, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward preprocess: delta[h][t] = <dO[t,h,:], O[t,h,:]>.
// ---------------------------------------------------------------------------


template <int D, bool BF16>
__global__ __launch_bounds__(256) void delta_kernel(DeltaArgs a) {
  constexpr int TPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / TPR;
  const int c = (int)(gid - r * TPR);
  const bool ok = r < (int64_t)a.heads * a.tokens;
  float acc = 0.f;
  if (ok) {
    const int h = (int)(r / a.tokens);
    const int64_t t = r - (int64_t)h * a.tokens;
    const float* orow = a.out + (t * a.heads + h) * D + c * 8;
    const char* drow = (const char*)a.dout + ((t * a.do_st + (int64_t)h * a.do_sh) + c * 8) * (BF16 ? 2 : 4);
    float dv[8];
    unpack8(drow, BF16, dv);
    const f32x4 o0 = ((const f32x4*)orow)[0], o1 = ((const f32x4*)orow)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(dv[i], o0[i], fmaf(dv[4 + i], o1[i], acc));
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (ok && c == 0) a.delta[r] = acc;
}

hipError_t launch_delta(const DeltaArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.heads * a.tokens * (a.d / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (a.d == 128) {
    if (a.bf16) hipLaunchKernelGGL((delta_kernel<128, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((delta_kernel<128, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.bf16) hipLaunchKernelGGL((delta_kernel<64, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((delta_kernel<64, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Zigzag gather / scatter (LongVILA article, ZIGZAG-RINGATTN; rule: sequence
// b is cut into 2cp chunks of L_b/(2cp) rows and rank r keeps chunks r and
// 2cp-1-r).  Local row t of sequence b sits at local offset o = t - cu_l[b]
// with cu_l[b] = cu_g[b]/cp; its global row is
//   cu_g[b] + (o < C ? r*C + o : (2cp-1-r)*C + o - C),  C = L_b/(2cp).
// One thread moves 16 bytes; the rows of a (token, head) are contiguous.
// ---------------------------------------------------------------------------


__global__ __launch_bounds__(256) void partition_kernel(PartArgs a) {
  const int cpr = a.row_bytes >> 4;                 // 16-byte chunks per (token, head)
  const int64_t per_tok = (int64_t)cpr * a.heads;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = gid / per_tok;
  if (t >= a.local_tokens) return;
  const int64_t rem = gid - t * per_tok;
  const int h = (int)(rem / cpr);
  const int c = (int)(rem - (int64_t)h * cpr);
  // rows past the last sequence, or a cu_seqlens array that points outside
  // the global tensor, move nothing
  if ((int64_t)a.cu[a.nseq] <= t * a.cp) return;
  int64_t g = t;
  if (a.cp > 1) {
    // last b with cu[b] <= t*cp
    const int64_t key = t * a.cp;
    int lo = 0, hi = a.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)a.cu[mid] <= key) lo = mid; else hi = mid - 1;
    }
    const int64_t gb = a.cu[lo];
    const int64_t len = (int64_t)a.cu[lo + 1] - gb;
    const int64_t C = len / (2 * a.cp);
    const int64_t o = t - gb / a.cp;
    g = gb + (o < C ? (int64_t)a.rank * C + o : (int64_t)(2 * a.cp - 1 - a.rank) * C + (o - C));
  }
  if (g < 0 || g >= a.global_tokens) return;
  const int64_t ls = a.scatter ? t : g;   // source row
  const int64_t ld = a.scatter ? g : t;   // destination row
  const u32x4 v = *(const u32x4*)(a.src + ls * a.src_st + h * a.src_sh + c * 16);
  *(u32x4*)(a.dst + ld * a.dst_st + h * a.dst_sh + c * 16) = v;
}

hipError_t launch_partition(const PartArgs& a, hipStream_t stream) {
  const int64_t threads = a.local_tokens * a.heads * (a.row_bytes >> 4);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(partition_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cpattn
