// Retained attention mass: the quality measure of a key-block selection.
//
// "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis",
// section 4 "Analysis" (Figure 3: retained attention mass of token-wise Top-K,
// fresh block-wise selection, cross-scale reuse and a sliding window; "Pattern
// Persistence across Clip Boundaries": against random blocks) and section 1
// (the gap to the token-wise bound split into blockization and scoring terms).
// With w_ts the dense softmax weight of query t on key s (every real key):
//
//   block_mass_*        M[i, j] = sum over the real queries t of query block i
//                       and the real keys s of key block j of w_ts, from the
//                       dense log-sum-exp of each query (w_ts = exp(sigma q.k - lse_t));
//   selection_mass      the mean over the real queries of block i of the mass
//                       on the blocks of a CSR list, sum_j M[i, j] / n_real(i);
//   window_scores       minus the distance between block centres in key-sequence
//                       position (query t is key L_text + L_ref + t): fed to the
//                       block selector it gives a sliding window;
//   token_topk_mass     per listed query, the mass of the retained key tokens plus
//                       the k_tokens largest candidate-token weights (the
//                       token-wise upper bound at the same key budget).
//
// block_mass_mfma_kernel (bf16, head_dim 128, 128-token blocks) has the shape of
// the first phase of the attention kernel: one workgroup of 4 wavefronts per
// query block, each wavefront 32 queries; 64-key sub-tiles of K go from global
// memory straight into double-buffered LDS (buffer_load_dwordx4 ... lds,
// XOR-swizzled 16-byte chunks), S^T = K Q^T by v_mfma_f32_32x32x16_bf16, then
// exp2 and a float32 sum per lane; at the end of a key block the lanes and the
// 4 wavefronts are summed in a fixed order (deterministic).  The other kernels
// are plain SIMT code.

#include "sparstar_internal.h"

#include <algorithm>
#include <type_traits>

namespace sparstar {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename T>
__device__ inline float to_f(T x) {
  return (float)x;
}

// ---------------------------------------------------------------- MFMA block mass

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kMB = 128;         // block size (queries and keys)
constexpr int kMD = 128;         // head_dim
constexpr int kSub = 64;         // keys per LDS sub-tile
constexpr int kTileBytes = kSub * kMD * 2;
constexpr int kBufferFlags = 0x00020000;  // word 3 of a raw buffer resource (32-bit data format)

__global__ __launch_bounds__(256, 2) void block_mass_mfma_kernel(MassArgs a, int per_xcd) {
  __shared__ __attribute__((aligned(16))) char k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char k_lds1[kTileBytes];
  __shared__ float red[2][4];
  lds_char* const kb[2] = {(lds_char*)k_lds0, (lds_char*)k_lds1};

  const Geometry& g = a.g;
  // XCD x = id mod 8 takes query blocks [x * per_xcd, (x + 1) * per_xcd) of every head.
  const int64_t kk = blockIdx.x / kXcds;
  const int64_t bh = kk / per_xcd;
  const int qi = (int)(blockIdx.x % kXcds) * per_xcd + (int)(kk - bh * per_xcd);
  if (qi >= g.n_q) return;  // uniform over the workgroup
  const int bi = (int)(bh / g.H), hi = (int)(bh - (int64_t)bi * g.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;

  const __bf16* qbase = static_cast<const __bf16*>(a.q) + bi * a.qs_b + hi * a.qs_h;
  const char* kbase = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.k) + bi * a.ks_b + hi * a.ks_h);

  // Q^T operand: lane holds query l32 of this wavefront, features 16 ks + 8 hl .. +8.
  const int64_t qrow = (int64_t)qi * kMB + wave * 32 + l32;
  const bool q_valid = qrow < g.L_q;
  bf16x8 qf[kMD / 16];
#pragma unroll
  for (int ks = 0; ks < kMD / 16; ++ks) {
    const uint4 raw =
        q_valid ? *reinterpret_cast<const uint4*>(qbase + qrow * a.qs_t + ks * 16 + hl * 8) : make_uint4(0, 0, 0, 0);
    __builtin_memcpy(&qf[ks], &raw, 16);
  }
  const float c = a.sigma * kLog2e;
  // Queries past the end contribute nothing: their offset is +inf, so every weight is 0.
  const float mc = q_valid ? a.lse[bh * g.L_q + qrow] * kLog2e : INFINITY;

  // Direct-to-LDS staging, one buffer resource per sub-tile (range = its real rows;
  // rows past the end read as zeros).  Wavefront w, pass t fills rows 16t + 4w .. +4;
  // lane i writes row + i/16 at physical chunk i%16, holding logical chunk (i%16) ^ (row & 15).
  const int st_row0 = 4 * wave + (lane >> 4);
  const uint32_t ks_b = (uint32_t)a.ks_t * 2u;
  const uint32_t k_thr = (uint32_t)st_row0 * ks_b + (uint32_t)(((lane & 15) ^ (st_row0 & 15)) * 16);
  auto load_sub = [&](int t, lds_char* buf) {
    // Sub-tile t covers keys [64 t, min(64 t + 64, L_k)); t past the end loads nothing.
    const int64_t first_key = (int64_t)t * kSub;
    const int len = (int)max<int64_t>(0, min<int64_t>(kSub, g.L_k - first_key));
    const char* first = kbase + (size_t)(len > 0 ? first_key : 0) * ks_b;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(first), (short)0, (int)((uint32_t)len * ks_b), kBufferFlags);
    lds_char* const ldsb = buf + 4 * wave * (kMD * 2);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, ldsb + p * 16 * (kMD * 2), 16, p * 16u * ks_b + k_thr, 0, 0, 0);
  };
  const uint32_t k_row = l32 * (kMD * 2), k_sw = hl ^ (l32 & 15);
  auto k_frag = [&](lds_char* buf, int kt, int ks) -> bf16x8 {
    typedef const __attribute__((address_space(3))) bf16x8* lds_bf16x8;
    return *(lds_bf16x8)(buf + kt * 32 * (kMD * 2) + k_row + (((2 * ks) ^ k_sw) << 4));
  };

  // Sub-tiles in key order: block j is sub-tiles 2j (even step, buffer 0) and 2j + 1
  // (odd step, buffer 1; empty when the last block holds at most 64 keys).  The
  // loads are unconditional (past the end they have an empty range) and each
  // step's buffers are fixed, so the compiler can tell which LDS buffer every
  // load writes and never waits for a load before reading the other buffer.
  const int n_sub = 2 * g.n_k;
  float* mrow = a.mass + (bh * g.n_q + qi) * (int64_t)g.n_k;
  float acc = 0.f;
  auto step = [&](int t, auto par) {
    constexpr int P = decltype(par)::value;
    lds_char* const cur = kb[P];
    load_sub(t + 1, kb[P ^ 1]);
    f32x16 s[2];
#pragma unroll
    for (int ks = 0; ks < kMD / 16; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(cur, kt, ks), qf[ks], ks == 0 ? f32x16{} : s[kt],
                                                        0, 0, 0);
    // Register r of tile kt holds key 64 t + 32 kt + 8 (r / 4) + 4 hl + r % 4.
    const int len = (int)max<int64_t>(0, min<int64_t>(kSub, g.L_k - (int64_t)t * kSub));
    float part = 0.f;
    if (len == kSub) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) part += __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -mc));
    } else {
      const int lim = len - 4 * hl;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + (r >> 2) * 8 + (r & 3) < lim) part += __builtin_amdgcn_exp2f(fmaf(s[kt][r], c, -mc));
    }
    acc += part;
    const int j = t >> 1;
    if (P == 1) {
      // End of key block j: this wavefront's total into red[j & 1][wave].
      const float w = wave_sum(acc);
      if (lane == 0) red[j & 1][wave] = w;
      acc = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (P == 1 && tid == 0) mrow[j] = (red[j & 1][0] + red[j & 1][1]) + (red[j & 1][2] + red[j & 1][3]);
  };
  load_sub(0, kb[0]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < n_sub; t += 2) {
    step(t, std::integral_constant<int, 0>());
    step(t + 1, std::integral_constant<int, 1>());
  }
}

// ---------------------------------------------------------------- SIMT block mass

// One workgroup of 256 threads per (batch, head, query block), thread = query (the
// first b threads); keys staged through LDS in float32, 32 at a time.
template <typename T, int D>
__global__ __launch_bounds__(256) void block_mass_simt_kernel(MassArgs a) {
  constexpr int kChunk = 32;
  __shared__ float ks[kChunk][D + 1];
  __shared__ float red[256];
  const Geometry& g = a.g;
  const int64_t row = blockIdx.x;  // bh * n_q + i
  const int64_t bh = row / g.n_q;
  const int i = (int)(row - bh * g.n_q);
  const int bi = (int)(bh / g.H), hi = (int)(bh - (int64_t)bi * g.H);
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)i * g.b + tid;
  const bool valid = tid < g.b && t < g.L_q;
  const T* qp = static_cast<const T*>(a.q) + bi * a.qs_b + hi * a.qs_h;
  const T* kp = static_cast<const T*>(a.k) + bi * a.ks_b + hi * a.ks_h;
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = valid ? to_f(qp[t * a.qs_t + d]) : 0.f;
  const float c = a.sigma * kLog2e;
  const float mc = valid ? a.lse[bh * g.L_q + t] * kLog2e : INFINITY;
  float* mrow = a.mass + row * (int64_t)g.n_k;

  for (int j = 0; j < g.n_k; ++j) {
    const int64_t k0 = (int64_t)j * g.b;
    const int len = (int)min<int64_t>(g.b, g.L_k - k0);
    float sum = 0.f;
    for (int c0 = 0; c0 < len; c0 += kChunk) {
      const int n = min(kChunk, len - c0);
      __syncthreads();
      for (int e = tid; e < n * D; e += blockDim.x) ks[e / D][e % D] = to_f(kp[(k0 + c0 + e / D) * a.ks_t + e % D]);
      __syncthreads();
      for (int u = 0; u < n; ++u) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(q[d], ks[u][d], dot);
        sum += __builtin_amdgcn_exp2f(fmaf(dot, c, -mc));
      }
    }
    // Fixed-order tree over the threads of the workgroup.
    red[tid] = valid ? sum : 0.f;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    if (tid == 0) mrow[j] = red[0];
  }
}

// ---------------------------------------------------------------- selection mass

// One wavefront per row; entries outside [0, col_idx_len) or [0, n_k) are skipped.
__global__ __launch_bounds__(256) void selection_mass_kernel(SelMassArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  int64_t beg = a.row_ptr[row], end = a.row_ptr[row + 1];
  if (beg < 0) beg = 0;
  if (end > a.col_idx_len) end = a.col_idx_len;
  const float* m = a.mass + row * (int64_t)a.n_k;
  float s = 0.f;
  for (int64_t p = beg + lane; p < end; p += 64) {
    const int j = a.col_idx[p];
    if (j >= 0 && j < a.n_k) s += m[j];
  }
  s = wave_sum(s);
  const int i = (int)(row % a.n_q);
  const int64_t n_real = min<int64_t>(a.b, a.L_q - (int64_t)i * a.b);
  if (lane == 0) a.out[row] = s / (float)n_real;
}

// ---------------------------------------------------------------- window scores

__global__ __launch_bounds__(256) void window_scores_kernel(float* out, int64_t total, int n_q, int n_k, int b,
                                                            int64_t offset) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int j = (int)(e % n_k);
    const int i = (int)((e / n_k) % n_q);
    // centres j*b + b/2 and offset + i*b + b/2: the halves cancel
    out[e] = -fabsf((float)((int64_t)(j - i) * b - offset));
  }
}

// ---------------------------------------------------------------- token-wise Top-K

// One workgroup (256 threads) per listed query.  Every pass recomputes the weights
// w_s = exp2(sigma log2(e) q.k_s - lse log2(e)): 16 lanes per key, one 16-byte load
// each, summed over the 16 lanes.  Candidate weights are ranked by their float32 bit
// patterns (non-negative floats order like their bits): four 8-bit MSB-first radix
// passes find the exact k-th largest, a last pass sums the weights above it.
template <typename T, int D>
__global__ __launch_bounds__(256) void token_topk_kernel(TopkArgs a) {
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte load
  constexpr int LPK = D / VEC;          // lanes per key (16 for bf16 / D=128, ...)
  constexpr int KPI = 256 / LPK;        // keys per workgroup iteration
  __shared__ uint32_t hist[256];
  __shared__ float fred[256];
  __shared__ uint32_t ured[256];
  __shared__ uint32_t sel[2];
  const Geometry& g = a.g;
  const int64_t qidx = a.rows[blockIdx.x];  // bh * L_q + t
  if (qidx < 0 || qidx >= (int64_t)g.B * g.H * g.L_q) {  // uniform over the workgroup
    if (threadIdx.x == 0) a.out[blockIdx.x] = __builtin_nanf("");
    return;
  }
  const int64_t bh = qidx / g.L_q, t = qidx - bh * g.L_q;
  const int bi = (int)(bh / g.H), hi = (int)(bh - (int64_t)bi * g.H);
  const int tid = threadIdx.x, sub = tid % LPK, kslot = tid / LPK;
  const T* qp = static_cast<const T*>(a.q) + bi * a.qs_b + hi * a.qs_h + t * a.qs_t + sub * VEC;
  const T* kp = static_cast<const T*>(a.k) + bi * a.ks_b + hi * a.ks_h + sub * VEC;
  float qv[VEC];
  {
    const uint4 raw = *reinterpret_cast<const uint4*>(qp);
    T tmp[VEC];
    __builtin_memcpy(tmp, &raw, 16);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[e] = to_f(tmp[e]);
  }
  const float c = a.sigma * kLog2e, mc = a.lse[qidx] * kLog2e;
  const int64_t L_k = g.L_k, keep = min<int64_t>(a.keep_tokens, L_k);
  const int64_t n_cand = L_k - keep;
  const int64_t K = min<int64_t>(a.k_tokens, n_cand);

  // Weight of key s, valid in every lane of the key's 16-lane group.
  auto weight = [&](int64_t s) -> float {
    const uint4 raw = *reinterpret_cast<const uint4*>(kp + s * a.ks_t);
    T tmp[VEC];
    __builtin_memcpy(tmp, &raw, 16);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) d = fmaf(qv[e], to_f(tmp[e]), d);
#pragma unroll
    for (int o = LPK / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, LPK);
    return __builtin_amdgcn_exp2f(fmaf(d, c, -mc));
  };
  auto block_fsum = [&](float x) -> float {  // fixed-order sum over the workgroup
    fred[tid] = x;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
      if (tid < o) fred[tid] += fred[tid + o];
      __syncthreads();
    }
    const float r = fred[0];
    __syncthreads();
    return r;
  };
  auto block_usum = [&](uint32_t x) -> uint32_t {
    ured[tid] = x;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
      if (tid < o) ured[tid] += ured[tid + o];
      __syncthreads();
    }
    const uint32_t r = ured[0];
    __syncthreads();
    return r;
  };

  // Retained tokens: their full mass.
  float kept = 0.f;
  for (int64_t s0 = 0; s0 < keep; s0 += KPI) {
    const int64_t s = s0 + kslot;
    const float w = s < keep ? weight(s) : 0.f;
    if (sub == 0) kept += w;
  }
  const float kept_sum = block_fsum(kept);

  float top = 0.f;
  if (K > 0) {
    uint32_t prefix = 0, mask = 0;
    uint32_t k_rem = (uint32_t)K;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int64_t s0 = keep; s0 < L_k; s0 += KPI) {
        const int64_t s = s0 + kslot;
        if (s < L_k) {
          const uint32_t u = __float_as_uint(weight(s));
          if (sub == 0 && (u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      if (tid == 0) {
        // Bin of the k_rem-th largest among the keys that match the prefix.
        uint32_t above = 0;
        int d = 255;
        for (; d > 0; --d) {
          if (above + hist[d] >= k_rem) break;
          above += hist[d];
        }
        sel[0] = (uint32_t)d;
        sel[1] = k_rem - above;
      }
      __syncthreads();
      prefix |= sel[0] << shift;
      mask |= 255u << shift;
      k_rem = sel[1];
      __syncthreads();
    }
    // prefix is now the bit pattern of the K-th largest candidate weight.
    float s_gt = 0.f;
    uint32_t n_gt = 0;
    for (int64_t s0 = keep; s0 < L_k; s0 += KPI) {
      const int64_t s = s0 + kslot;
      if (s < L_k) {
        const float w = weight(s);
        if (sub == 0 && __float_as_uint(w) > prefix) {
          s_gt += w;
          ++n_gt;
        }
      }
    }
    const float sum_gt = block_fsum(s_gt);
    const uint32_t cnt_gt = block_usum(n_gt);
    top = sum_gt + (float)((uint32_t)K - cnt_gt) * __uint_as_float(prefix);
  }
  if (tid == 0) a.out[blockIdx.x] = kept_sum + top;
}

}  // namespace

hipError_t launch_block_mass(const MassArgs& a, hipStream_t s) {
  const Geometry& g = a.g;
  const int64_t rows = (int64_t)g.B * g.H * g.n_q;
  if (rows == 0 || g.n_k == 0) return hipSuccess;
  const bool mfma = a.dtype == 0 && g.D == kMD && g.b == kMB && a.small_extent;
  if (mfma) {
    const int per_xcd = (g.n_q + kXcds - 1) / kXcds;
    const int64_t grid = (int64_t)g.B * g.H * per_xcd * kXcds;
    if (grid > 0xffffffffll) return hipErrorInvalidValue;
    hipLaunchKernelGGL(block_mass_mfma_kernel, dim3((unsigned)grid), dim3(256), 0, s, a, per_xcd);
  } else {
    if (rows > 0xffffffffll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)rows), block(256);
    if (a.dtype == 0 && g.D == 128)
      hipLaunchKernelGGL((block_mass_simt_kernel<__bf16, 128>), grid, block, 0, s, a);
    else if (a.dtype == 0)
      hipLaunchKernelGGL((block_mass_simt_kernel<__bf16, 64>), grid, block, 0, s, a);
    else if (g.D == 128)
      hipLaunchKernelGGL((block_mass_simt_kernel<float, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((block_mass_simt_kernel<float, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_selection_mass(const SelMassArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const int64_t blocks = (a.rows + 3) / 4;
  if (blocks > 0xffffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(selection_mass_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_window_scores(float* out, int64_t bh, int n_q, int n_k, int b, int64_t offset, hipStream_t s) {
  const int64_t total = bh * n_q * n_k;
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(window_scores_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, total, n_q, n_k, b, offset);
  return hipGetLastError();
}

hipError_t launch_token_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.n_rows > 0xffffffffll) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.n_rows), block(256);
  if (a.dtype == 0 && a.g.D == 128)
    hipLaunchKernelGGL((token_topk_kernel<__bf16, 128>), grid, block, 0, s, a);
  else if (a.dtype == 0)
    hipLaunchKernelGGL((token_topk_kernel<__bf16, 64>), grid, block, 0, s, a);
  else if (a.g.D == 128)
    hipLaunchKernelGGL((token_topk_kernel<float, 128>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((token_topk_kernel<float, 64>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace sparstar
