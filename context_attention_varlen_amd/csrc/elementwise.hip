// HBM-bound kernels: LSE merge, backward preprocess (delta), zigzag
// gather/scatter.
#include "common.h"

namespace cpattn {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// LSE merge.  Ring Attention ("Scaling Video Training with Parallelism",
// section 2) produces one partial (out, lse) per key/value block; two partial
// results over disjoint key sets combine as the softmax over their union:
//   lse' = m + log(exp(lse - m) + exp(lse_p - m)),  m = max(lse, lse_p)
//   out' = exp(lse - lse') out + exp(lse_p - lse') out_p
// A row with lse_p = -inf passes through (out is neither read nor written),
// except that a row whose running lse is still -inf is set to 0 (the result
// over no keys): the running output needs no initialisation.
// (A variant keeping 4 rows in flight per thread, with a quarter of the
// threads, measured slower: 72 -> 84 us per long-tail merge.)
// ---------------------------------------------------------------------------


// Streaming loads and stores bypass cache residency (nontemporal): every
// byte is touched once.
template <class T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <class T>
__device__ __forceinline__ void st_nt(T v, T* p) { __builtin_nontemporal_store(v, p); }

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// 4 elements of a row at element offset e: fp32, or bf16 widened to fp32
template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* row, int e) {
  if (BF16) {
    const u32x2 raw = ld_nt((const u32x2*)((const uint16_t*)row + e));
    return f32x4{__uint_as_float(raw[0] << 16), __uint_as_float(raw[0] & 0xffff0000u),
                 __uint_as_float(raw[1] << 16), __uint_as_float(raw[1] & 0xffff0000u)};
  }
  return ld_nt((const f32x4*)((const float*)row + e));
}

// Rows are visited token-major (r = t*H + h), the order of `out` and of the
// partial in memory, so both stream contiguously; thread c of a row owns
// elements [4c, 4c + 4). The head-major LSE reads of 16 consecutive tokens
// share one cache line.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / TPR;
  const int c = (int)(gid - r * TPR);
  if (r >= (int64_t)a.heads * a.tokens) return;
  const int64_t t = r / a.heads;
  const int h = (int)(r - t * a.heads);
  const int64_t li = (int64_t)h * a.tokens + t;
  const float lp = a.lsep[li];
  const float lo = a.lse[li];
  float* o = a.out + r * D + 4 * c;
  if (lp == -INFINITY) {
    // nothing to add; a row not yet merged (running lse -inf) becomes the
    // result over no keys, 0, so the running output needs no initialisation
    if (lo == -INFINITY) st_nt(f32x4{0.f, 0.f, 0.f, 0.f}, (f32x4*)o);
    return;
  }
  const void* prow = (const char*)a.op + (t * a.op_st + (int64_t)h * a.op_sh) * (BF16 ? 2 : 4);
  const f32x4 p = load4<BF16>(prow, 4 * c);
  f32x4 v;
  float nl;
  if (lo == -INFINITY) {
    v = p;
    nl = lp;
  } else {
    const float m = fmaxf(lo, lp);
    const float eo = __expf(lo - m), ep = __expf(lp - m);
    const float s = eo + ep;
    nl = m + __logf(s);
    const float inv = 1.f / s;
    const float w_o = eo * inv, w_p = ep * inv;
    v = ld_nt((const f32x4*)o);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = w_o * v[i] + w_p * p[i];
  }
  st_nt(v, (f32x4*)o);
  if (c == 0) a.lse[li] = nl;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.heads * a.tokens * (a.d / 4);
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
// Fill: the ring's starting state (out = 0, lse = -inf, the merge identity)
// and zeroed gradient accumulators.  One thread stores 16 bytes,
// nontemporal (every byte is written once and not read back soon); the
// last count mod 4 values are stored singly by the first threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_kernel(float* dst, int64_t count, float value) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nvec = count >> 2;
  if (i < nvec) st_nt(f32x4{value, value, value, value}, (f32x4*)dst + i);
  const int64_t tail = count - (nvec << 2);
  if (i < tail) dst[(nvec << 2) + i] = value;
}

hipError_t launch_fill(float* dst, int64_t count, float value, hipStream_t stream) {
  const int64_t threads = std::max<int64_t>(count >> 2, 3);
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, dst, count, value);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward preprocess: delta[h][t] = <dO[t,h,:], O[t,h,:]>.
// ---------------------------------------------------------------------------


// Token-major rows (the order of `out` and dO in memory), 4 elements per thread.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void delta_kernel(DeltaArgs a) {
  constexpr int TPR = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / TPR;
  const int c = (int)(gid - r * TPR);
  const bool ok = r < (int64_t)a.heads * a.tokens;
  const int64_t t = r / a.heads;
  const int h = (int)(r - t * a.heads);
  float acc = 0.f;
  if (ok) {
    const void* drow = (const char*)a.dout + (t * a.do_st + (int64_t)h * a.do_sh) * (BF16 ? 2 : 4);
    const f32x4 d4 = load4<BF16>(drow, 4 * c);
    const f32x4 o4 = ld_nt((const f32x4*)(a.out + r * D + 4 * c));
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(d4[i], o4[i], acc);
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (ok && c == 0) a.delta[(int64_t)h * a.tokens + t] = acc;
}

hipError_t launch_delta(const DeltaArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.heads * a.tokens * (a.d / 4);
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
// Under the height/width split (LongCat-Video context-parallel page) local
// row o of a frames x H x W sample is row o mod (th*tw) of frame o/(th*tw)
// inside the rank's grid cell of th x tw tokens.
// Under the balanced teacher-forcing split ("Scaling Video Training with
// Parallelism", section 4) local row o of a sequence is, with m = N/cp time
// chunks per rank, row o mod B of the rank's (o/B mod m)-th time chunk in the
// clean stream (o < mB) or the noisy stream.
// A workgroup moves the rows of a few consecutive local tokens: their global
// rows are resolved once per token (binary search over cu_seqlens) into LDS,
// then every thread keeps kPartK 16-byte nontemporal loads in flight over the
// (token, head, 16-byte chunk) triples; the rows of a (token, head) are
// contiguous, so consecutive threads touch consecutive bytes.
// ---------------------------------------------------------------------------

constexpr int kPartThreads = 256;
constexpr int kPartK = 8;                                  // 16-byte chunks in flight per thread
constexpr int kPartMaxTok = kPartThreads;                  // local rows per workgroup, at most

// Global row of local row t, or -1 when the row moves nothing (past the last
// sequence, or a cu_seqlens array that points outside the global tensor).
__device__ int64_t part_global_row(const PartArgs& a, int64_t t) {
  if ((int64_t)a.cu[a.nseq] <= t * a.cp) return -1;
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
    const int64_t o = t - gb / a.cp;
    if (a.hw_h > 0) {
      // height/width split: rank r's grid cell (r / sw, r mod sw) of every
      // frame, cell rows top to bottom, each left to right
      const int64_t th = a.hw_h / a.hw_sh, tw = a.hw_w / a.hw_sw, cell = th * tw;
      const int64_t f = o / cell, rem = o - f * cell;
      const int64_t hh = rem / tw, ww = rem - hh * tw;
      const int64_t rh = a.rank / a.hw_sw, rw = a.rank - rh * a.hw_sw;
      g = gb + (f * a.hw_h + rh * th + hh) * a.hw_w + rw * tw + ww;
    } else if (a.tf_b > 0) {
      // balanced teacher forcing: [clean chunks of the rank ; noisy chunks],
      // N/cp time chunks of B rows in each stream
      const int64_t B = a.tf_b, m = a.tf_n / a.cp;
      const int64_t blk = o / B;
      const bool noisy = blk >= m;
      const int64_t c = tf_rank_chunk(a.rank, (int32_t)(noisy ? blk - m : blk), a.cp);
      g = gb + (noisy ? B * a.tf_n : 0) + c * B + (o - blk * B);
    } else {
      const int64_t C = len / (2 * a.cp);
      g = gb + (o < C ? (int64_t)a.rank * C + o : (int64_t)(2 * a.cp - 1 - a.rank) * C + (o - C));
    }
  }
  return (g < 0 || g >= a.global_tokens) ? -1 : g;
}

__global__ __launch_bounds__(kPartThreads) void partition_kernel(PartArgs a) {
  __shared__ int64_t s_row[kPartMaxTok];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * a.tok_per_block;
  const int ntok = (int)min((int64_t)a.tok_per_block, a.local_tokens - t0);
  if (tid < ntok) s_row[tid] = part_global_row(a, t0 + tid);
  __syncthreads();
  const int cmask = (1 << a.cpr_shift) - 1;
  const unsigned per_tok = (unsigned)a.heads << a.cpr_shift;   // 16-byte chunks per token
  const unsigned total = (unsigned)ntok * per_tok;
  for (unsigned base = 0; base < total; base += kPartThreads * kPartK) {
    u32x4 v[kPartK];
    int64_t dofs[kPartK];
#pragma unroll
    for (int k = 0; k < kPartK; ++k) {
      const unsigned i = base + k * kPartThreads + tid;
      dofs[k] = -1;
      if (i < total) {
        const unsigned tt = i / per_tok, rem = i - tt * per_tok;
        const int h = (int)(rem >> a.cpr_shift), c = (int)(rem & cmask);
        const int64_t g = s_row[tt];
        if (g >= 0) {
          const int64_t t = t0 + tt;
          const int64_t ls = a.scatter ? t : g;   // source row
          const int64_t ld = a.scatter ? g : t;   // destination row
          v[k] = ld_nt((const u32x4*)(a.src + ls * a.src_st + h * a.src_sh + c * 16));
          dofs[k] = ld * a.dst_st + h * a.dst_sh + c * 16;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPartK; ++k)
      if (dofs[k] >= 0) st_nt(v[k], (u32x4*)(a.dst + dofs[k]));
  }
}

hipError_t launch_partition(PartArgs a, hipStream_t stream) {
  if (a.local_tokens <= 0 || a.heads <= 0) return hipSuccess;
  int shift = 0;
  while ((16 << shift) < a.row_bytes) ++shift;
  if ((16 << shift) != a.row_bytes) return hipErrorInvalidValue;   // rows are 128, 256 or 512 bytes
  a.cpr_shift = shift;
  const int64_t per_tok = (int64_t)a.heads << shift;
  a.tok_per_block = (int)std::max<int64_t>(1, std::min<int64_t>(kPartMaxTok, kPartThreads * kPartK / per_tok));
  const int64_t blocks = (a.local_tokens + a.tok_per_block - 1) / a.tok_per_block;
  hipLaunchKernelGGL(partition_kernel, dim3((unsigned)blocks), dim3(kPartThreads), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Ulysses sequence <-> head exchange on one device ("Scaling Video Training
// with Parallelism", SP landscape: DeepSpeed-Ulysses shards the sequence and
// exchanges all-to-all around attention so that every member holds all
// tokens of a head group).  With the shards resident, each shard's block of
// rows moves as one strided copy; one thread moves 16 bytes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void head_copy_kernel(HeadCopyArgs a) {
  const int cpr = a.row_bytes >> 4;
  const int64_t per_tok = (int64_t)cpr * a.heads;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = gid / per_tok;
  if (t >= a.tokens) return;
  const int64_t rem = gid - t * per_tok;
  const int h = (int)(rem / cpr);
  const int c = (int)(rem - (int64_t)h * cpr);
  const u32x4 v = ld_nt((const u32x4*)(a.src + (a.src_row0 + t) * a.src_st + (int64_t)(a.src_h0 + h) * a.src_sh + c * 16));
  st_nt(v, (u32x4*)(a.dst + (a.dst_row0 + t) * a.dst_st + (int64_t)(a.dst_h0 + h) * a.dst_sh + c * 16));
}

hipError_t launch_head_copy(const HeadCopyArgs& a, hipStream_t stream) {
  const int64_t threads = a.tokens * a.heads * (a.row_bytes >> 4);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(head_copy_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cpattn
