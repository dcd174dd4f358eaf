// Fused linear cross-entropy kernels for gfx950 and their launch sequence.
//
// Forward ("Chunked and Fused Cross-Entropy", llms.blog, "Mathematical
// Mechanics" steps 1-2; lesson 27 "Trick 1" and "Trick 2"):
//   k_label_scan   valid-token count D, invalid-label count, scale g/D, and a
//                  per-token-block "has a valid label" flag
//   k_fwd_lse      logit tiles Z = W_tile . X_tile^T on MFMA, reduced on chip
//                  with the running max / sum-exp recurrence into one
//                  (m, l, z_y, sum z) partial per (vocab split, token)
//   k_lse_merge    fixed-order merge of the partials -> LSE_i and l_i, plus a
//                  fixed-order per-256-token loss sum
//   k_loss_final   fixed-order sum of those block sums, / D (NaN on bad labels)
// Backward, per logit block of C_N tokens x C_V vocabulary columns in fixed
// order (lesson 27 "Trick 2": recompute, then the two matmul-backward products):
//   k_bwd_dz       recompute the block's logits on MFMA and write
//                  dZ = softmax - q (unscaled) to the scratch block
//   k_bwd_grad     dW[block vocab] (=|+=) s * dZ^T X[block tokens]   (M = vocab)
//                  dX[block tokens] (=|+=) s * dZ W[block vocab]     (M = tokens)
// No floating-point atomics: every sum has a fixed order, so results are
// bitwise reproducible.
#include "fce_kernels.h"

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "fce_gemm.h"

namespace fce {
namespace {

__device__ __forceinline__ bool label_ok(int y, int ignore, int V) {
  return y != ignore && y >= 0 && y < V;
}

// (m, l, t, z) merge: running max m, sum l of exp(z - m), target logit t,
// logit sum z.  Either side may be empty (m = -inf, l = 0).
__device__ __forceinline__ void lse_merge(float& m, float& l, float& t, float& z, float m2,
                                          float l2, float t2, float z2) {
  const float mn = fmaxf(m, m2);
  if (mn != -INFINITY) l = l * hw_exp2((m - mn) * kLog2e) + l2 * hw_exp2((m2 - mn) * kLog2e);
  m = mn;
  t += t2;
  z += z2;
}

__device__ __forceinline__ void lse_merge(floatx4& a, const floatx4& b) {
  float m = a[0], l = a[1], t = a[2], z = a[3];
  lse_merge(m, l, t, z, b[0], b[1], b[2], b[3]);
  a = floatx4{m, l, t, z};
}

// ---------------------------------------------------------------- label scan
// reduction: 0 mean (D = max(N_valid, 1)), 1 sum (D = 1), 2 none (D = 1, and
// the upstream gradient is applied per token by the dZ kernel).
__global__ __launch_bounds__(1024) void k_label_scan(const int32_t* __restrict__ labels, int N,
                                                     int V, int ignore, int reduction,
                                                     const float* __restrict__ grad, Ctrl* ctrl,
                                                     int32_t* flags, int CN, int nblocks) {
  __shared__ int s_valid[1024], s_bad[1024];
  const int tid = threadIdx.x;
  for (int c = tid; c < nblocks; c += 1024) flags[c] = 0;
  __syncthreads();
  int nv = 0, nb = 0;
  for (int i = tid; i < N; i += 1024) {
    const int y = labels[i];
    if (label_ok(y, ignore, V)) {
      ++nv;
      flags[i / CN] = 1;
    } else if (y != ignore) {
      ++nb;
    }
  }
  s_valid[tid] = nv;
  s_bad[tid] = nb;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) {
      s_valid[tid] += s_valid[tid + s];
      s_bad[tid] += s_bad[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int n_valid = s_valid[0];
    const float D = (reduction != 0) ? 1.0f : static_cast<float>(n_valid > 0 ? n_valid : 1);
    const float g = (grad && reduction != 2) ? grad[0] : 1.0f;
    ctrl->n_valid = n_valid;
    ctrl->n_invalid = s_bad[0];
    ctrl->scale_fwd = D;  // the loss is divided by D
    ctrl->scale_bwd = g / D;
  }
}

// ------------------------------------------------------------------ forward
// Four consecutive elements of a row, rounded to T (bf16: nearest even).
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  floatx4 v = {a, b, c, d};
  *reinterpret_cast<floatx4*>(p) = v;
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const floatx4 f = {a, b, c, d};
  *reinterpret_cast<bf16x4*>(p) = __builtin_convertvector(f, bf16x4);
}

// Global-memory byte pointer.
typedef __attribute__((address_space(1))) char gchar;

// The same address in scalar registers as a global pointer (the caller
// guarantees that p is wave-uniform), so that loads and stores address it as
// a scalar base plus a 32-bit lane offset.
template <typename P>
__device__ __forceinline__ gchar* wave_uniform(P* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  return reinterpret_cast<gchar*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// 16-byte non-temporal stores at base + off bytes, global or through a
// buffer resource.  The staged epilogues write whole row segments that this
// kernel never reads back (dZ is read by the next launches, dX and dW are
// outputs), so they are marked streaming: at 8192 x 4096 x 128256 that took
// dZ from 6.82 to 6.76 ms and dX from 6.52 to 6.40 ms per step.  The buffer
// form passes the whole offset in the vector register and a constant 0 as
// the scalar offset: with a register scalar offset, a VALU write of the data
// registers right after the store was seen to reach the last lanes' copy of
// the first word, and the compiler only separates the two when the scalar
// offset is a constant.
__device__ __forceinline__ void store16(gchar* base, uint32_t off, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<__attribute__((address_space(1))) u32x4*>(base + off));
}
constexpr int kBufNonTemporal = 2;  // cache-policy bit of the buffer store (nt)
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kBufNonTemporal);
}

// Buffer resource at a wave-uniform base with a record count the caller has
// already clamped to [0, 2^31 - 1]; every field goes through readfirstlane,
// so it is legal wherever the compiler keeps the inputs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, uint32_t n) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  void* bs = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(
      bs, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(n)), 0x00020000);
}

// a + b (b wave-uniform) computed where it is used: kept out of loop-invariant
// hoisting, which would hold one register per use across the whole loop.
__device__ __forceinline__ uint32_t add_at_use(uint32_t a, uint32_t b) {
  uint32_t r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "v"(b), "v"(a));
  return r;
}

// Waits until this wave's LDS reads have returned their data, and keeps the
// compiler from moving memory operations across (a staging region is
// written through float or bf16 pointers and read back through 16-byte
// vectors, types that alias analysis would let it reorder).  Used before a
// staging region is rewritten.
__device__ __forceinline__ void lds_reads_done() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <typename T>
struct FwdArgs {
  const T* X;
  const T* W;
  const int32_t* labels;
  int N, H, V, ignore;
  int tok_tiles, voc_tiles, splits, group_m;
  int64_t n_pad;
  floatx4* part;  // [splits][n_pad]: (m, l, z_y, sum z)
  T* zout;        // STORE: logits [N][ldz] in T, columns up to the tile coverage
  int64_t ldz;
};

// STORE: also write every logit tile, rounded to T, to zout (the logits of
// the store-logits variant).  Columns past V hold 0 (W rows past V load as
// zeros), so a row is written up to the vocabulary tile coverage.
// STREAM (bf16, H % 128 == 0): all vocabulary tiles of the split as one DMA
// stream; otherwise one GEMM tile and its epilogue per vocabulary tile.
template <class C, bool SMOOTH, bool STORE, bool STREAM>
__global__ __launch_bounds__(C::NT) void k_fwd_lse(FwdArgs<typename C::Elem> a) {
  typedef typename C::Elem T;
  FCE_DMA_STAGES(lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  int tt, sp;
  grouped_tile(xcd_remap(blockIdx.x, a.tok_tiles * a.splits), a.tok_tiles, a.splits, a.group_m,
               tt, sp);
  const int n0 = tt * C::BN;
  const int vt_begin = static_cast<int>(static_cast<int64_t>(sp) * a.voc_tiles / a.splits);
  const int vt_end = static_cast<int>(static_cast<int64_t>(sp + 1) * a.voc_tiles / a.splits);
  const Opnd<T> A{a.W, a.H, a.V, a.H};  // rows: vocabulary
  const Opnd<T> B{a.X, a.H, a.N, a.H};  // rows: tokens

  typedef AccMap<C> Map;
  int yv[C::FN];
  float rm[C::FN], rl[C::FN], rt[C::FN], rz[C::FN];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int tok = n0 + wn * C::WTN + fn * C::NB + Map::col(lane);
    const int y = tok < a.N ? a.labels[tok] : a.ignore;
    yv[fn] = label_ok(y, a.ignore, a.V) ? y : -1;
    rm[fn] = -INFINITY;
    rl[fn] = rt[fn] = rz[fn] = 0.0f;
  }

  // Running (max, sum-exp, target logit, logit sum) update of one logit tile
  // whose rows are the vocabulary entries m0 .. m0+BM-1.  FULL: no row past
  // V (every tile but the last), so the loops take no masks.
  auto update = [&](auto full_c, const Acc<C>& acc, int m0) {
    constexpr bool FULL = decltype(full_c)::value;
    const int vbase = m0 + wm * C::WTM;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      if constexpr (STORE) {
        const int tok = n0 + wn * C::WTN + fn * C::NB + Map::col(lane);
        if (tok < a.N) {
          T* zr = a.zout + static_cast<int64_t>(tok) * a.ldz + vbase;
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int g = 0; g < Map::NGRP; ++g)
              store4(zr + fm * C::MB + Map::row(lane, g), acc.v[fm][fn][4 * g],
                     acc.v[fm][fn][4 * g + 1], acc.v[fm][fn][4 * g + 2], acc.v[fm][fn][4 * g + 3]);
        }
      }
      // Element i of block fm sits at row vbase + row(lane, 0) + off with
      // off = fm MB + row(lane, i / 4) - row(lane, 0) + i % 4, the same for
      // every lane.  A token's label lies in this wave's WTM rows of one
      // tile in about WTM / V of them: the search for the target logit runs
      // only when some lane's does (a wave-uniform branch).
      const int rel = yv[fn] - vbase - Map::row(lane, 0);
      if (__ballot(static_cast<unsigned>(yv[fn] - vbase) < static_cast<unsigned>(C::WTM)) != 0) {
        float tg = 0.0f;
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int i = 0; i < C::NV; ++i) {
            const int off = fm * C::MB + Map::row(lane, i >> 2) - Map::row(lane, 0) + (i & 3);
            tg += (rel == off) ? acc.v[fm][fn][i] : 0.0f;
          }
        rt[fn] += tg;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int i = 0; i < C::NV; ++i) {
          const int off = fm * C::MB + Map::row(lane, i >> 2) - Map::row(lane, 0) + (i & 3);
          if (FULL || vbase + Map::row(lane, 0) + off < a.V) tmax = fmaxf(tmax, acc.v[fm][fn][i]);
        }
      const float mnew = fmaxf(rm[fn], tmax);
      if (mnew == -INFINITY) continue;  // nothing valid seen yet in this lane
      // exp(z - m) as exp2(z log2e - m log2e): one FMA per element
      const float mb = mnew * kLog2e;
      float s = 0.0f, zs = 0.0f;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int i = 0; i < C::NV; ++i) {
          const int off = fm * C::MB + Map::row(lane, i >> 2) - Map::row(lane, 0) + (i & 3);
          const float z = acc.v[fm][fn][i];
          const bool ok = FULL || vbase + Map::row(lane, 0) + off < a.V;
          // fp32: exp2((z - m) log2e), exact near the max, so each term's
          // relative error does not grow with |m|; bf16 keeps the one-FMA form
          float e;
          if constexpr (sizeof(T) == 4)
            e = hw_exp2((z - mnew) * kLog2e);
          else
            e = hw_exp2(__builtin_fmaf(z, kLog2e, -mb));
          s += ok ? e : 0.0f;
          if (SMOOTH) zs += ok ? z : 0.0f;
        }
      rl[fn] = rl[fn] * hw_exp2((rm[fn] - mnew) * kLog2e) + s;
      rm[fn] = mnew;
      rz[fn] += zs;
      // one token column at a time: keeps the accumulator copies it needs,
      // not the whole tile's, in vector registers
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto lse_update = [&](const Acc<C>& acc, int m0) {
    if (m0 + C::BM <= a.V)
      update(std::true_type{}, acc, m0);
    else
      update(std::false_type{}, acc, m0);
  };
  if constexpr (STREAM) {
    static_assert(sizeof(T) == 2, "the stream is bf16");
    gemm_stream_pp<C>(A, B, vt_begin, vt_end, n0, a.H, lds, tid, lse_update);
  } else {
    Acc<C> acc;
    for (int vt = vt_begin; vt < vt_end; ++vt) {
      const int m0 = vt * C::BM;
      gemm_any<C, true, true>(acc, A, B, m0, n0, a.H, lds, tid);
      lse_update(acc, m0);
    }
  }

  // the 64 / NB lanes that share a column (l, l ^ NB, ...) hold disjoint rows
  // of it: merge them pairwise (the merge is symmetric, so both lanes of a
  // pair end with the same bits)
#pragma unroll
  for (int sh = C::NB; sh < 64; sh <<= 1) {
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const float m2 = __shfl_xor(rm[fn], sh);
      const float l2 = __shfl_xor(rl[fn], sh);
      const float t2 = __shfl_xor(rt[fn], sh);
      const float z2 = __shfl_xor(rz[fn], sh);
      lse_merge(rm[fn], rl[fn], rt[fn], rz[fn], m2, l2, t2, z2);
    }
  }
  // then the WAVES_M waves that share these token columns, in fixed order
  static_assert(C::WAVES_M * C::BN * sizeof(floatx4) <= 32768, "reduction fits one stage");
  floatx4* red = reinterpret_cast<floatx4*>(lds.s[0]);  // [WAVES_M][BN]; free after gemm_any
  if (lane < C::NB) {
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      floatx4 st = {rm[fn], rl[fn], rt[fn], rz[fn]};
      red[wm * C::BN + wn * C::WTN + fn * C::NB + lane] = st;
    }
  }
  __syncthreads();
  if (wm == 0 && lane < C::NB) {
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int col = wn * C::WTN + fn * C::NB + lane;
      floatx4 st = red[col];
      for (int w = 1; w < C::WAVES_M; ++w) {
        const floatx4 o = red[w * C::BN + col];
        lse_merge(st, o);
      }
      const int tok = n0 + col;
      if (tok < a.N) a.part[static_cast<int64_t>(sp) * a.n_pad + tok] = st;
    }
  }
}

// The forward over grid workgroups: the stream when the operands allow it.
template <class C, bool SMOOTH, bool STORE>
void launch_fwd_lse(const FwdArgs<typename C::Elem>& fa, int grid, hipStream_t st) {
  if constexpr (sizeof(typename C::Elem) == 2) {
    if (fa.H % 128 == 0) {
      k_fwd_lse<C, SMOOTH, STORE, true><<<grid, C::NT, 0, st>>>(fa);
      return;
    }
  }
  k_fwd_lse<C, SMOOTH, STORE, false><<<grid, C::NT, 0, st>>>(fa);
}

// Per token: LSE from the split partials, the loss term
// l = LSE - (1-eps) z_y - (eps/V) sum z + alpha LSE^2, and a fixed-order sum
// per block of kLossBlock tokens.  tok_loss (reduction none) receives l, 0
// for an ignored row and NaN for a label outside [0, V).
__global__ __launch_bounds__(kLossBlock) void k_lse_merge(
    const floatx4* __restrict__ part, int splits, int64_t n_pad, const int32_t* __restrict__ labels,
    int N, int V, int ignore, float eps, float zloss, float* __restrict__ lse,
    float* __restrict__ blockloss, float* __restrict__ tok_loss, float2* __restrict__ stat) {
  __shared__ float s_red[kLossBlock];
  const int tok = blockIdx.x * kLossBlock + threadIdx.x;
  float term = 0.0f;
  if (tok < N) {
    const int y = labels[tok];
    if (label_ok(y, ignore, V)) {
      floatx4 st = part[tok];
      for (int s = 1; s < splits; ++s) {
        const floatx4 o = part[static_cast<int64_t>(s) * n_pad + tok];
        lse_merge(st, o);
      }
      // LSE = m + log l, kept split as well (m, log2 l): the large part m
      // cancels exactly against the logits near the max, where the rounded
      // sum m + log l would carry an error of |LSE| 2^-25
      const float lg = hw_log2(st[1]);
      const float L = st[0] + lg * kLn2;
      lse[tok] = L;
      if (stat) stat[tok] = float2{st[0], lg};
      term = (st[0] - (1.0f - eps) * st[2]) + lg * kLn2;
      if (eps != 0.0f) term -= (eps / static_cast<float>(V)) * st[3];
      if (zloss != 0.0f) term += zloss * L * L;
      if (tok_loss) tok_loss[tok] = term;
    } else {
      lse[tok] = NAN;
      if (stat) stat[tok] = float2{0.0f, INFINITY};
      if (tok_loss) tok_loss[tok] = (y == ignore) ? 0.0f : NAN;
    }
  }
  s_red[threadIdx.x] = term;
  __syncthreads();
  for (int s = kLossBlock / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) s_red[threadIdx.x] += s_red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) blockloss[blockIdx.x] = s_red[0];
}

__global__ __launch_bounds__(256) void k_loss_final(const float* __restrict__ blockloss,
                                                    int nblocks, const Ctrl* __restrict__ ctrl,
                                                    float* __restrict__ loss) {
  __shared__ float s_red[256];
  float acc = 0.0f;
  for (int b = threadIdx.x; b < nblocks; b += 256) acc += blockloss[b];
  s_red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) s_red[threadIdx.x] += s_red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = ctrl->n_invalid > 0 ? NAN : s_red[0] / ctrl->scale_fwd;
}

// p[0 .. n) *= g[0], 16 bytes per thread and step (p 16-byte aligned; the
// last n % 4 elements one by one).
__global__ __launch_bounds__(256) void k_scale(float* __restrict__ p, int64_t n,
                                               const float* __restrict__ g) {
  const float s = g[0];
  const int64_t nv = n / 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t i0 = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  for (int64_t i = i0; i < nv; i += stride) {
    floatx4* q = reinterpret_cast<floatx4*>(p) + i;
    *q = *q * s;
  }
  if (i0 < n - 4 * nv) p[4 * nv + i0] *= s;
}

__global__ void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0.0f;
}

// ------------------------------------------------------------ backward: dZ
template <typename T>
struct DzArgs {
  const T* X;  // X + tok0 * H
  const T* W;  // W + voc0 * H
  const int32_t* labels;  // labels + tok0
  const float* lse;       // lse + tok0
  int ntok, nvoc, voc0, H, V, ignore;
  float eps, zloss;
  const float* gtok;  // per-token upstream gradient (reduction none) + tok0, or NULL
  int voc_tiles, tok_tiles, group_m;
  T* dz;
  int64_t ldz;
  const int32_t* flag;  // this token block's "has a valid label" flag
  uint8_t* keep;        // FILTER: [tok_tiles][voc_tiles] tile kept (1) or skipped (0)
  // fp32: the forward's split row statistics (m, log2 l) + tok0, or NULL to
  // take the exponent from the LSE alone
  const float2* stat;
};

// Gradient filtering ("Cut Cross-Entropy", llms.blog, "Apple Cut
// Cross-Entropy (CCE)"): a dZ tile is skipped when every softmax value in it
// is below 2^-12 and it holds no label of its tokens (the target term is
// never dropped).
constexpr float kFilterP = 0.000244140625f;  // 2^-12

// FILTER: also decide whether the tile is kept (see kFilterP), record it in
// keep[], and store only kept tiles.
template <class C, bool KFULL, bool FILTER>
__global__ __launch_bounds__(C::NT) void k_bwd_dz(DzArgs<typename C::Elem> a) {
  typedef typename C::Elem T;
  int vt, tt;
  grouped_tile(xcd_remap(blockIdx.x, a.voc_tiles * a.tok_tiles), a.voc_tiles, a.tok_tiles,
               a.group_m, vt, tt);
  if (*a.flag == 0) {  // every label of this token block is ignored
    if (FILTER && threadIdx.x == 0) a.keep[tt * a.voc_tiles + vt] = 0;
    return;
  }
  FCE_DMA_STAGES(lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int m0 = vt * C::BM, n0 = tt * C::BN;
  const Opnd<T> A{a.W, a.H, a.nvoc, a.H};
  const Opnd<T> B{a.X, a.H, a.ntok, a.H};
  Acc<C> acc;
  gemm_any<C, true, true, KFULL>(acc, A, B, m0, n0, a.H, lds, tid);

  typedef AccMap<C> Map;
  const float eps_v = a.eps / static_cast<float>(a.V);
  const float one_m_eps = 1.0f - a.eps;
  // FULL: no column past nvoc in this tile (workgroup-uniform; only the
  // block's last vocabulary tile can have them), so no column masks.
  auto epilogue = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    bool keep = false;  // FILTER: this lane's vote
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int tl = n0 + wn * C::WTN + fn * C::NB + Map::col(lane);
      const int y = tl < a.ntok ? a.labels[tl] : a.ignore;
      const bool valid = tl < a.ntok && label_ok(y, a.ignore, a.V);
      const float L = valid ? a.lse[tl] : 0.0f;
      // d(alpha LSE^2)/dz = 2 alpha LSE p; reduction none scales the row by
      // g_i.  dZ = (e zf - eps/V) g_i with e = exp2(z log2e - LSE log2e) is
      // two FMAs; an ignored row takes exponent offset +inf (e = 0) and
      // g_i = 0, so its dZ is exactly 0.
      const float gi = valid ? (a.gtok ? a.gtok[tl] : 1.0f) : 0.0f;
      const float lb = valid ? L * kLog2e : INFINITY;
      // fp32: exp2((z - m) log2e - log2 l) with the forward's split
      // statistics (or m = LSE, log2 l = 0 without them): the subtraction is
      // exact near the max, so p keeps its accuracy at large |LSE|
      float sm = 0.0f, slg = INFINITY;
      if constexpr (sizeof(T) == 4) {
        if (valid) {
          const float2 sv = a.stat ? a.stat[tl] : float2{L, 0.0f};
          sm = sv.x;
          slg = sv.y;
        }
      }
      auto expo = [&](float z) -> float {
        if constexpr (sizeof(T) == 4)
          return hw_exp2(__builtin_fmaf(z - sm, kLog2e, -slg));
        else
          return hw_exp2(__builtin_fmaf(z, kLog2e, -lb));
      };
      const float c1 = (1.0f + 2.0f * a.zloss * L) * gi;
      const float c0 = -eps_v * gi;
      const int vrow = m0 + wm * C::WTM + Map::row(lane, 0);  // row of element 0
      T* row = a.dz + static_cast<int64_t>(tl) * a.ldz + vrow;
      // The one-hot term, (1 - eps) g_i at the label column.  Element i of
      // block fm sits at row vrow + off(fm, i), off the same for every lane.
      // The label lies in this wave's WTM rows of the tile for few tokens,
      // so only then does the loop test for it (chosen once per column by a
      // wave-uniform branch); subtracting 0 elsewhere would not change a bit.
      const int rel = valid ? y - a.voc0 - vrow : -1 - C::WTM;
      const float t = one_m_eps * gi;
      if constexpr (FILTER) {
        // dZ in place of the accumulators and this lane's vote; the tile is
        // stored below if any lane of the workgroup votes to keep it
        keep |= valid && static_cast<unsigned>(y - a.voc0 - m0) < static_cast<unsigned>(C::BM);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int i = 0; i < C::NV; ++i) {
            const int off = fm * C::MB + Map::row(lane, i >> 2) - Map::row(lane, 0) + (i & 3);
            const bool ok = FULL || vrow + off < a.nvoc;
            const float e = expo(acc.v[fm][fn][i]);
            keep |= ok && e >= kFilterP;
            float d = __builtin_fmaf(e, c1, c0);
            d -= (rel == off) ? t : 0.0f;
            acc.v[fm][fn][i] = ok ? d : 0.0f;
          }
      } else {
        auto column = [&](auto label_c) {
          constexpr bool LABEL = decltype(label_c)::value;
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int g = 0; g < Map::NGRP; ++g) {
              const int off0 = fm * C::MB + Map::row(lane, g) - Map::row(lane, 0);
              float d[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                d[q] = __builtin_fmaf(expo(acc.v[fm][fn][4 * g + q]), c1, c0);
                if (LABEL) d[q] -= (rel == off0 + q) ? t : 0.0f;
                if (!FULL) d[q] = (vrow + off0 + q < a.nvoc) ? d[q] : 0.0f;
              }
              store4(row + off0, d[0], d[1], d[2], d[3]);
            }
        };
        if (__ballot(static_cast<unsigned>(rel + Map::row(lane, 0)) <
                     static_cast<unsigned>(C::WTM)) != 0)
          column(std::true_type{});
        else
          column(std::false_type{});
      }
    }
    return keep;
  };
  // (the filtered path rewrites the accumulators in place: one masked copy,
  // whose masks are all true in full tiles, keeps it in registers)
  bool keep;
  if (!FILTER && m0 + C::BM <= a.nvoc)
    keep = epilogue(std::true_type{});
  else
    keep = epilogue(std::false_type{});
  if constexpr (FILTER) {
    __shared__ int s_keep[C::NT / 64];
    const bool wave_keep = __ballot(keep) != 0;  // every lane votes
    if (lane == 0) s_keep[wave] = wave_keep;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < C::NT / 64; ++w) any |= s_keep[w];
    if (tid == 0) a.keep[tt * a.voc_tiles + vt] = static_cast<uint8_t>(any);
    if (!any) return;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int tl = n0 + wn * C::WTN + fn * C::NB + Map::col(lane);
      T* row = a.dz + static_cast<int64_t>(tl) * a.ldz;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int g = 0; g < Map::NGRP; ++g)
          store4(row + m0 + wm * C::WTM + fm * C::MB + Map::row(lane, g), acc.v[fm][fn][4 * g],
                 acc.v[fm][fn][4 * g + 1], acc.v[fm][fn][4 * g + 2], acc.v[fm][fn][4 * g + 3]);
    }
  }
}

// dZ as one DMA stream per workgroup (bf16, H % 128 == 0 and H >= 256, no
// filtering): one token tile against vocabulary tiles vt_begin .. vt_end-1
// of the block, the recompute of each logit tile on the ping-pong stream of
// gemm_stream_pp_st and its dZ epilogue in the memory phase of each wave
// group, so the K pipeline stays full across vocabulary tiles and one
// group's epilogue runs beside the other group's MFMAs.  Same dZ bits as
// k_bwd_dz: the per-token factors are computed once, before the stream,
// with the same expressions.
// FILTER: also cast the gradient-filtering votes (kFilterP): a wave whose
// part of a vocabulary tile holds a softmax value of at least 2^-12, or the
// label of one of its tokens, writes 1 to the tile's keep flag (zeroed
// before the launch; concurrent writers write the same byte).  Every tile is
// still stored, so a kept tile's dZ is whole.
template <class C, bool FILTER = false>
__global__ __launch_bounds__(C::NT) void k_bwd_dz_stream(DzArgs<bf16> a, int splits) {
  int tt, sp;
  grouped_tile(xcd_remap(blockIdx.x, a.tok_tiles * splits), a.tok_tiles, splits, a.group_m, tt,
               sp);
  if (*a.flag == 0) return;  // every label of this token block is ignored
  FCE_DMA_STAGES(lds);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: staging bases stay scalar
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int n0 = tt * C::BN;
  const int vt_begin = static_cast<int>(static_cast<int64_t>(sp) * a.voc_tiles / splits);
  const int vt_end = static_cast<int>(static_cast<int64_t>(sp + 1) * a.voc_tiles / splits);
  const Opnd<bf16> A{a.W, a.H, a.nvoc, a.H};
  const Opnd<bf16> B{a.X, a.H, a.ntok, a.H};
  typedef AccMap<C> Map;
  const float eps_v = a.eps / static_cast<float>(a.V);
  const float one_m_eps = 1.0f - a.eps;
  // Per token column of the tile, kept in LDS beside the four stages (so
  // that nothing live across the stream is spilled): the exponent offset
  // LSE log2e (+inf for an ignored row), dZ = exp * c1 + c0, the one-hot
  // term t at the label, and the label's row in the block (far out of range
  // for an ignored row).
  __shared__ float s_lb[C::BN], s_c1[C::BN], s_c0[C::BN], s_tk[C::BN];
  __shared__ int s_yv[C::BN];
  for (int c = tid; c < C::BN; c += C::NT) {
    const int tl = n0 + c;
    const int y = tl < a.ntok ? a.labels[tl] : a.ignore;
    const bool valid = tl < a.ntok && label_ok(y, a.ignore, a.V);
    const float L = valid ? a.lse[tl] : 0.0f;
    const float gi = valid ? (a.gtok ? a.gtok[tl] : 1.0f) : 0.0f;
    s_lb[c] = valid ? L * kLog2e : INFINITY;
    s_c1[c] = (1.0f + 2.0f * a.zloss * L) * gi;
    s_c0[c] = -eps_v * gi;
    s_tk[c] = one_m_eps * gi;
    s_yv[c] = valid ? y - a.voc0 : INT_MIN / 2;
  }
  __syncthreads();
  const int rbase = wm * C::WTM + Map::row(lane, 0);
  // bytes from a wave's strip origin to the end of its WTN token rows
  const uint32_t strip_bytes = static_cast<uint32_t>(
      min(static_cast<int64_t>(C::WTN) * a.ldz * 2, static_cast<int64_t>(0x7fffffff)));
  // Store staging: one 16-token column of a wave's WTM-row strip at a time
  // passes through LDS, so that each store writes 16-byte pieces of whole
  // token-row segments (2 WTM bytes) instead of 8-byte pieces scattered
  // over 16 rows.  Region wn serves the two waves of column wn, whose
  // epilogues are half a K step apart with a workgroup barrier between
  // them (and the LDS operations of a wave run in order).  Rows are padded
  // by 16 bytes, which spreads the writes of the 16 tokens over the banks.
  constexpr int kRowB = 2 * C::WTM, kPitch = kRowB + 16, kPieces = kRowB / 16;
  static_assert(C::NB == 16 && Map::NGRP == 1 && 64 % kPieces == 0, "staging geometry");
  __shared__ __attribute__((aligned(16))) char s_stage[C::WAVES_N][C::NB * kPitch];
  char* const stg = s_stage[wn];
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  auto epilogue = [&](auto full_c, const Acc<C>& acc, int m0) {
    constexpr bool FULL = decltype(full_c)::value;
    const int vrow = m0 + rbase;  // row of element 0
    bool vote = false;            // FILTER: this lane's vote for the tile
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int c = wn * C::WTN + fn * C::NB + Map::col(lane);
      const float lb = s_lb[c], c1 = s_c1[c], c0 = s_c0[c], tk = s_tk[c];
      const int rel = s_yv[c] - vrow;
      // the label of this token in the tile's BM rows (never for an
      // ignored row, whose label row is far out of range)
      if (FILTER) vote |= static_cast<unsigned>(s_yv[c] - m0) < static_cast<unsigned>(C::BM);
      auto column = [&](auto label_c) {
        constexpr bool LABEL = decltype(label_c)::value;
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
          const int off0 = fm * C::MB;
          floatx4 d;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float e = hw_exp2(__builtin_fmaf(acc.v[fm][fn][q], kLog2e, -lb));
            if (FILTER) vote |= (FULL || vrow + off0 + q < a.nvoc) && e >= kFilterP;
            float v = __builtin_fmaf(e, c1, c0);
            if (LABEL) v -= (rel == off0 + q) ? tk : 0.0f;
            if (!FULL) v = (vrow + off0 + q < a.nvoc) ? v : 0.0f;
            d[q] = v;
          }
          *reinterpret_cast<bf16x4*>(stg + Map::col(lane) * kPitch +
                                     2 * (off0 + Map::row(lane, 0))) =
              __builtin_convertvector(d, bf16x4);
        }
      };
      if (__ballot(static_cast<unsigned>(rel + Map::row(lane, 0)) <
                   static_cast<unsigned>(C::WTM)) != 0)
        column(std::true_type{});
      else
        column(std::false_type{});
      // the strip's 16 token rows, 64 / kPieces of them per store, through a
      // buffer resource based at this wave's strip of the tile, with 32-bit
      // lane offsets
      const __amdgpu_buffer_rsrc_t rs = make_rsrc_n(
          a.dz + static_cast<int64_t>(n0 + wn * C::WTN) * a.ldz + m0 + wm * C::WTM, strip_bytes);
      const uint32_t ldz_b = static_cast<uint32_t>(a.ldz) * 2u;
      const uint32_t voff = static_cast<uint32_t>(lane / kPieces) * ldz_b + 16u * (lane % kPieces);
      constexpr int NJ = C::NB * kPieces / 64;
      u32x4 v[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = j * (64 / kPieces) + lane / kPieces, piece = lane % kPieces;
        v[j] = *reinterpret_cast<const u32x4*>(stg + t * kPitch + 16 * piece);
      }
      lds_reads_done();  // before the next column's writes to the region
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        store16(rs, add_at_use(voff, static_cast<uint32_t>(fn * C::NB + j * (64 / kPieces)) * ldz_b),
                v[j]);
      // one token column at a time (keeps the live values of one column)
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FILTER) {
      if (__ballot(vote) != 0 && lane == 0) a.keep[tt * a.voc_tiles + m0 / C::BM] = 1;
    }
  };
  // the epilogue's stores per wave, every one unconditional (masked columns
  // store zeros)
  constexpr int kStores = C::FN * (C::NB * kPieces / 64);
  gemm_stream_pp_st<C, kStores>(A, B, vt_begin, vt_end, n0, a.H, lds, tid,
                             [&](const Acc<C>& acc, int m0) {
                               if (m0 + C::BM <= a.nvoc)
                                 epilogue(std::true_type{}, acc, m0);
                               else
                                 epilogue(std::false_type{}, acc, m0);
                             });
}

// ---------------------------------------------------- backward: dW and dX
template <typename T>
struct GradArgs {
  Opnd<T> A;  // dZ^T (dW) or dZ (dX)
  Opnd<T> B;  // X^T (dW) or W^T (dX), both MN-major
  int K;      // contraction length covered by the tile loop
  int m_valid, n_valid;
  int tm_tiles, tn_tiles, group_m;
  float* out;  // first output row of this block
  int64_t ldo;
  const Ctrl* ctrl;
  int accumulate;
  const int32_t* flag;
  // split over K (gridDim.y > 1): split z covers k in [z ksplit, (z+1) ksplit)
  // and writes its own output at out + z * split_stride
  int ksplit;
  int64_t split_stride;
  // FILTER: the kept K blocks (kMapBlock long) of output row tile tm are
  // klist[tm * list_ld + 0 .. kcount[tm]-1], ascending; korder lists the row
  // tiles by descending kept count (longest first)
  const int* klist;
  const int* kcount;
  int list_ld;
  const int* korder;
};

// The part of an operand from contraction index k0 on.
template <bool KMAJOR, typename T>
__device__ __forceinline__ Opnd<T> opnd_from_k(const Opnd<T>& o, int k0) {
  return Opnd<T>{o.p + (KMAJOR ? static_cast<int64_t>(k0) : static_cast<int64_t>(k0) * o.ld), o.ld,
                 o.mn_ext, o.k_ext - k0};
}

// fp32 output of one full bf16 tile (16 x 16 blocks), scaled by s, stored
// or added to the values in place, through LDS: each wave stages 32 rows of
// its WTM x WTN strip at a time in a region of its own within the DMA stages
// (free once the K loop has drained), then moves whole row segments of WTN
// floats with 16-byte loads and stores.  The lane-per-element epilogue moves
// 4-byte pieces over four rows per instruction instead.  Same arithmetic, in
// the same order, as that epilogue: out = old + s acc, or s acc.
template <class C>
__device__ __forceinline__ void store_grad_tile_staged(const Acc<C>& acc, float s, float* tile,
                                                       int64_t ldo, bool accumulate,
                                                       const DmaStages& st, int wave, int lane) {
  typedef AccMap<C> Map;
  constexpr int kRows = 32, kRowB = 4 * C::WTN, kPitch = kRowB + 16, kPieces = kRowB / 16;
  constexpr int kRowsPer = 64 / kPieces;  // rows per 16-byte instruction
  static_assert(C::MB == 16 && C::NB == 16 && Map::NGRP == 1 && C::WTM % kRows == 0 &&
                    64 % kPieces == 0 && 2 * kRows * kPitch <= 32768 && C::NT / 64 <= 8,
                "staging geometry: two waves per 32 KiB stage");
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int w2 = wave >> 1;  // (constant indices: the stage table is not an array in memory)
  char* const reg = (w2 == 0 ? st.s[0] : w2 == 1 ? st.s[1] : w2 == 2 ? st.s[2] : st.s[3]) +
                    (wave & 1) * (kRows * kPitch);
  gchar* const sb = wave_uniform(tile + static_cast<int64_t>(wm * C::WTM) * ldo + wn * C::WTN);
  const uint32_t ldo_b = static_cast<uint32_t>(ldo) * 4u;
  const uint32_t voff = static_cast<uint32_t>(lane / kPieces) * ldo_b + 16u * (lane % kPieces);
#pragma unroll
  for (int rr = 0; rr < C::WTM / kRows; ++rr) {
    // element (fm, fn, q): row fm MB + row(lane, 0) + q, column fn NB + col(lane)
#pragma unroll
    for (int j = 0; j < kRows / C::MB; ++j)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float*>(reg + (j * C::MB + Map::row(lane, 0) + q) * kPitch +
                                    4 * (fn * C::NB + Map::col(lane))) =
              s * acc.v[rr * (kRows / C::MB) + j][fn][q];
    constexpr int NI = kRows / kRowsPer;
    floatx4 v[NI], old[NI];
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const uint32_t soff = static_cast<uint32_t>(rr * kRows + t * kRowsPer) * ldo_b;
      old[t] = accumulate
                   ? *reinterpret_cast<const __attribute__((address_space(1))) floatx4*>(sb + voff + soff)
                          : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int t = 0; t < NI; ++t)
      v[t] = *reinterpret_cast<const floatx4*>(
          reg + (t * kRowsPer + lane / kPieces) * kPitch + 16 * (lane % kPieces));
    lds_reads_done();  // before the next round's writes to the region
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const uint32_t soff = static_cast<uint32_t>(rr * kRows + t * kRowsPer) * ldo_b;
      const floatx4 o = accumulate ? old[t] + v[t] : v[t];
      store16(sb, voff + soff, __builtin_bit_cast(u32x4, o));
    }
  }
}

// Xt[h][n] = X[n][h] for n < N, 0 for N <= n < ldt: X^T for the dW product
// as (dW)^T = X^T dZ, whose K-major A operand it is.  64 x 64 tiles through
// LDS; 16-byte loads along h and 16-byte stores along n.
__global__ __launch_bounds__(256) void k_transpose_x(const bf16* __restrict__ X, int N, int H,
                                                     bf16* __restrict__ Xt, int64_t ldt) {
  __shared__ uint16_t t[64][64 + 2];
  const int n0 = blockIdx.x * 64, h0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  // load: 64 rows (n) x 8 vectors of 8 (h); thread -> (row, vector)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + 256 * r;
    const int n = n0 + i / 8, hv = 8 * (i % 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < N && h0 + hv < H) v = *reinterpret_cast<const u32x4*>(X + static_cast<int64_t>(n) * H + h0 + hv);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[i / 8][hv + 2 * j] = static_cast<uint16_t>(v[j] & 0xffffu);
      t[i / 8][hv + 2 * j + 1] = static_cast<uint16_t>(v[j] >> 16);
    }
  }
  __syncthreads();
  // store: 64 rows (h) x 8 vectors of 8 (n)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + 256 * r;
    const int h = h0 + i / 8, nv = 8 * (i % 8);
    if (h >= H || n0 + nv >= ldt) continue;
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = static_cast<uint32_t>(t[nv + 2 * j][i / 8]) |
             (static_cast<uint32_t>(t[nv + 2 * j + 1][i / 8]) << 16);
    *reinterpret_cast<u32x4*>(Xt + static_cast<int64_t>(h) * ldt + n0 + nv) = v;
  }
}

// The transposed counterpart of store_grad_tile_staged, for a tile computed
// as (out)^T: the tile's M runs along the columns of out and its N along the
// rows, out element (n, m) at tile + n ldo + m.  A lane holds 4 consecutive m
// of one n, so each wave stages one 16-row block of n (its 16 x WTM floats)
// at a time with 16-byte LDS writes, then moves whole row segments of WTM
// floats with 16-byte loads and stores.  Same arithmetic, in the same order:
// out = old + s acc, or s acc.
template <class C>
__device__ __forceinline__ void store_grad_tile_staged_t(const Acc<C>& acc, float s, float* tile,
                                                         int64_t ldo, bool accumulate,
                                                         const DmaStages& st, int wave, int lane) {
  typedef AccMap<C> Map;
  constexpr int kRowB = 4 * C::WTM, kPitch = kRowB + 16, kPieces = kRowB / 16;
  constexpr int kRowsPer = 64 / kPieces;  // rows per 16-byte instruction
  constexpr int NI = C::NB / kRowsPer;
  static_assert(C::MB == 16 && C::NB == 16 && Map::NGRP == 1 && 64 % kPieces == 0 &&
                    2 * C::NB * kPitch <= 32768 && C::NT / 64 <= 8,
                "staging geometry: two waves per 32 KiB stage");
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int w2 = wave >> 1;  // (constant indices: the stage table is not an array in memory)
  char* const reg = (w2 == 0 ? st.s[0] : w2 == 1 ? st.s[1] : w2 == 2 ? st.s[2] : st.s[3]) +
                    (wave & 1) * (C::NB * kPitch);
  gchar* const sb = wave_uniform(tile + static_cast<int64_t>(wn * C::WTN) * ldo + wm * C::WTM);
  const uint32_t ldo_b = static_cast<uint32_t>(ldo) * 4u;
  const uint32_t voff = static_cast<uint32_t>(lane / kPieces) * ldo_b + 16u * (lane % kPieces);
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    // element (fm, fn, q): m = fm MB + row(lane, 0) + q, n = fn NB + col(lane)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const floatx4 v = {s * acc.v[fm][fn][0], s * acc.v[fm][fn][1], s * acc.v[fm][fn][2],
                         s * acc.v[fm][fn][3]};
      *reinterpret_cast<floatx4*>(reg + Map::col(lane) * kPitch +
                                  4 * (fm * C::MB + Map::row(lane, 0))) = v;
    }
    floatx4 v[NI], old[NI];
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const uint32_t soff = static_cast<uint32_t>(fn * C::NB + t * kRowsPer) * ldo_b;
      old[t] = accumulate
                   ? *reinterpret_cast<const __attribute__((address_space(1))) floatx4*>(sb + voff + soff)
                   : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int t = 0; t < NI; ++t)
      v[t] = *reinterpret_cast<const floatx4*>(
          reg + (t * kRowsPer + lane / kPieces) * kPitch + 16 * (lane % kPieces));
    lds_reads_done();  // before the next block's writes to the region
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const uint32_t soff = static_cast<uint32_t>(fn * C::NB + t * kRowsPer) * ldo_b;
      const floatx4 o = accumulate ? old[t] + v[t] : v[t];
      store16(sb, voff + soff, __builtin_bit_cast(u32x4, o));
    }
  }
}

// Tile (tm, tn) of a gradient product's grid (tm_tiles x tn_tiles) for
// workgroup `bid`: the XCD-aware order, or with FILTER and rows of unequal
// kept length, the longest rows first in dispatch order.
template <class C, bool FILTER>
__device__ __forceinline__ void grad_tile_index(const GradArgs<typename C::Elem>& a, int bid,
                                                int& tm, int& tn) {
  if (FILTER && a.kcount[a.korder[0]] != a.kcount[a.korder[a.tm_tiles - 1]]) {
    tm = a.korder[bid / a.tn_tiles];
    tn = bid % a.tn_tiles;
  } else {
    grouped_tile(xcd_remap(bid, a.tm_tiles * a.tn_tiles), a.tm_tiles, a.tn_tiles, a.group_m, tm,
                 tn);
  }
}

// Output tile (tm, tn) of a gradient product, split z of nz over the
// contraction.  TRANS: the tile is (out)^T, out element (n, m) at
// out + n ldo + m (the dW product computed as X^T dZ).
template <class C, bool A_KMAJOR, bool FILTER, bool TRANS>
__device__ __forceinline__ void grad_tile_at(const GradArgs<typename C::Elem>& a, int tm, int tn,
                                             int z, int nz, const DmaStages& lds) {
  typedef typename C::Elem T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const bool skip = (*a.flag == 0);  // all labels of the token block ignored: dZ = 0
  if (skip && a.accumulate) return;
  Opnd<T> A = a.A, B = a.B;
  int K = a.K;
  float* out = a.out;
  if (nz > 1) {
    const int k0 = z * a.ksplit;
    A = opnd_from_k<A_KMAJOR>(A, k0);
    B = opnd_from_k<false>(B, k0);
    K = min(a.ksplit, a.K - k0);
    out += static_cast<int64_t>(z) * a.split_stride;
  }
  Acc<C> acc;
  if constexpr (FILTER) {
    static_assert(sizeof(T) == 2 && C::BM == kMapBlock && C::BN == kMapBlock,
                  "filtered products: bf16 tiles one kept block long");
    const int cnt = skip ? 0 : a.kcount[tm];
    if (cnt == 0 && a.accumulate) return;
    if (cnt == 0)
      zero_acc(acc);
    else if (cnt == (K + kMapBlock - 1) / kMapBlock)  // every block kept: the plain K loop
      gemm_any<C, A_KMAJOR, false, true>(acc, A, B, m0, n0, K, lds, tid);
    else
      gemm_tile_dma<C, A_KMAJOR, false, true, true>(acc, A, B, m0, n0, cnt * kMapBlock, lds, tid,
                                                    a.klist + tm * a.list_ld);
  } else if (skip) {
    zero_acc(acc);
  } else {
    // K is the token count (dW, no K-major operand) or the block's vocabulary
    // coverage, a whole number of tiles (dX)
    gemm_any<C, A_KMAJOR, false, true>(acc, A, B, m0, n0, K, lds, tid);
  }
  typedef AccMap<C> Map;
  const float s = a.ctrl->scale_bwd;
  // Output element (fm, fn, i) of this lane: row m0 + wm WTM + fm MB +
  // row(lane, i/4) + i%4, column n0 + wn WTN + fn NB + col(lane).  Per slab of
  // SLAB block rows, all loads of the old values are issued before any use,
  // so their latencies overlap.
  constexpr int SLAB = (C::MB >= 32) ? 1 : 32 / C::MB;
  static_assert(C::FM % SLAB == 0, "slabs of block rows");
  const int rbase = wm * C::WTM;
  const int cbase = wn * C::WTN + Map::col(lane);
  const bool full = m0 + C::BM <= a.m_valid && n0 + C::BN <= a.n_valid;
  float* tile = TRANS ? out + static_cast<int64_t>(n0) * a.ldo + m0
                      : out + static_cast<int64_t>(m0) * a.ldo + n0;
  if constexpr (sizeof(T) == 2) {
    if (full) {
      if constexpr (TRANS)
        store_grad_tile_staged_t<C>(acc, s, tile, a.ldo, a.accumulate != 0, lds, wave, lane);
      else
        store_grad_tile_staged<C>(acc, s, tile, a.ldo, a.accumulate != 0, lds, wave, lane);
      return;
    }
  }
#pragma unroll
  for (int f0 = 0; f0 < C::FM; f0 += SLAB) {
    float old[SLAB][C::FN][C::NV];
    bool ok[SLAB][C::FN][C::NV];
#pragma unroll
    for (int j = 0; j < SLAB; ++j)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int i = 0; i < C::NV; ++i) {
          const int r = rbase + (f0 + j) * C::MB + Map::row(lane, i >> 2) + (i & 3);
          const int c = cbase + fn * C::NB;
          ok[j][fn][i] = full || (m0 + r < a.m_valid && n0 + c < a.n_valid);
          old[j][fn][i] = 0.0f;
          if (a.accumulate && ok[j][fn][i])
            old[j][fn][i] = TRANS ? tile[static_cast<int64_t>(c) * a.ldo + r]
                                  : tile[static_cast<int64_t>(r) * a.ldo + c];
        }
#pragma unroll
    for (int j = 0; j < SLAB; ++j)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int i = 0; i < C::NV; ++i) {
          const int r = rbase + (f0 + j) * C::MB + Map::row(lane, i >> 2) + (i & 3);
          const int c = cbase + fn * C::NB;
          if (ok[j][fn][i])
            tile[TRANS ? static_cast<int64_t>(c) * a.ldo + r : static_cast<int64_t>(r) * a.ldo + c] =
                old[j][fn][i] + s * acc.v[f0 + j][fn][i];
        }
  }
}

// Tile `bid` of a gradient product's grid (see grad_tile_index).
template <class C, bool A_KMAJOR, bool FILTER, bool TRANS>
__device__ __forceinline__ void grad_tile(const GradArgs<typename C::Elem>& a, int bid, int z,
                                          int nz, const DmaStages& lds) {
  int tm, tn;
  grad_tile_index<C, FILTER>(a, bid, tm, tn);
  grad_tile_at<C, A_KMAJOR, FILTER, TRANS>(a, tm, tn, z, nz, lds);
}

// One gradient product: a grid of tm_tiles x tn_tiles workgroups, by nz
// splits of the contraction along y.
template <class C, bool A_KMAJOR, bool FILTER, bool TRANS = false>
__global__ __launch_bounds__(C::NT) void k_bwd_grad(GradArgs<typename C::Elem> a) {
  FCE_DMA_STAGES(lds);
  grad_tile<C, A_KMAJOR, FILTER, TRANS>(a, blockIdx.x, blockIdx.y, gridDim.y, lds);
}

// Both gradient products of one logit block in one launch (bf16): they read
// the same dZ block and write disjoint outputs, so their tiles share one
// grid.  The dW tiles take n_dw consecutive workgroup ids and the dX tiles
// n_dx per split z of dx_splits over the vocabulary; the longer kind of tile
// comes first (dx_first), so the short ones fill in behind it.  One grid
// lets the ragged last wave of either product fill with the other's tiles,
// and leaves one launch boundary per block instead of two.
template <class C, bool DW_KMAJOR, bool DW_TRANS>
__global__ __launch_bounds__(C::NT) void k_bwd_grad_pair(GradArgs<bf16> gw, GradArgs<bf16> gx,
                                                         int n_dw, int n_dx, int dx_splits,
                                                         int dx_first) {
  FCE_DMA_STAGES(lds);
  const int b = blockIdx.x;
  const int n_x = n_dx * dx_splits;
  const bool is_dw = dx_first ? b >= n_x : b < n_dw;
  if (is_dw) {
    grad_tile<C, DW_KMAJOR, false, DW_TRANS>(gw, dx_first ? b - n_x : b, 0, 1, lds);
  } else {
    const int r = dx_first ? b : b - n_dw;
    grad_tile<C, true, false, false>(gx, r % n_dx, r / n_dx, dx_splits, lds);
  }
}

// The filtered products of one logit block in one launch, dX tiles first
// when theirs is the longer contraction.  A dW tile whose vocabulary tile
// keeps every token block is computed as the exact path computes it, the
// (h, v) tile of (dW)^T = X^T dZ on the ping-pong loop (use_t: X^T is at
// hand, gt describes that product); every other dW tile as dZ^T X over its
// kept token blocks.  When every vocabulary tile keeps every token block
// (korder lists them by descending count), the dW tiles also take the exact
// path's tile order.
template <class C>
__global__ __launch_bounds__(C::NT) void k_bwd_grad_pair_filt(GradArgs<bf16> gw, GradArgs<bf16> gt,
                                                              GradArgs<bf16> gx, int n_dw,
                                                              int n_dx, int dx_first, int use_t) {
  FCE_DMA_STAGES(lds);
  const int b = blockIdx.x;
  const bool is_dw = dx_first ? b >= n_dx : b < n_dw;
  if (is_dw) {
    const int loc = dx_first ? b - n_dx : b;
    const int full = (gw.K + kMapBlock - 1) / kMapBlock;
    if (use_t && *gw.flag != 0 && gw.kcount[gw.korder[gw.tm_tiles - 1]] == full) {
      // every dW tile keeps every token block: the exact path's product, in
      // its tile order (groups of H-tile rows)
      grad_tile<C, true, false, true>(gt, loc, 0, 1, lds);
      return;
    }
    int tm, tn;  // vocabulary tile, H tile
    grad_tile_index<C, true>(gw, loc, tm, tn);
    if (use_t && *gw.flag != 0 && gw.kcount[tm] == full)
      grad_tile_at<C, true, false, true>(gt, tn, tm, 0, 1, lds);
    else
      grad_tile_at<C, false, true, false>(gw, tm, tn, 0, 1, lds);
  } else {
    grad_tile<C, true, true, false>(gx, dx_first ? b : b - n_dw, 0, 1, lds);
  }
}

// Kept-block lists of one logit block for the filtered products: per token
// tile (rows of dX) the kept vocabulary tiles, per vocabulary tile (rows of
// dW) the kept token tiles, ascending.  One wave per list: 64 flags at a
// time, compacted with a ballot and a population count.  stats[0] += kept
// tiles, stats[1] += all tiles of the block.
__global__ __launch_bounds__(64) void k_filter_lists(const uint8_t* __restrict__ keep, int tt,
                                                     int vt, int* __restrict__ rowlist,
                                                     int* __restrict__ rowcnt,
                                                     int* __restrict__ collist,
                                                     int* __restrict__ colcnt,
                                                     unsigned long long* __restrict__ stats) {
  const int i = blockIdx.x, lane = threadIdx.x;
  const bool is_row = i < tt;
  const int len = is_row ? vt : tt;  // entries of this list
  int* out = is_row ? rowlist + i * vt : collist + (i - tt) * tt;
  int c = 0;
  for (int base = 0; base < len; base += 64) {
    const int e = base + lane;
    const bool k = e < len && keep[is_row ? i * vt + e : e * vt + (i - tt)] != 0;
    const unsigned long long m = __ballot(k);
    if (k) out[c + __popcll(m & ((1ull << lane) - 1ull))] = e;
    c += __popcll(m);
  }
  if (lane == 0) {
    (is_row ? rowcnt[i] : colcnt[i - tt]) = c;
    if (is_row) atomicAdd(&stats[0], static_cast<unsigned long long>(c));
    if (i == 0) atomicAdd(&stats[1], static_cast<unsigned long long>(tt) * vt);
  }
}

// Row tiles of the two filtered products by descending kept count (ties by
// index): rank of row i = rows with a larger count, or an equal count and a
// smaller index.  One workgroup; counts of at most a few hundred rows.
__global__ __launch_bounds__(256) void k_filter_order(const int* __restrict__ rowcnt, int tt,
                                                      int* __restrict__ roworder,
                                                      const int* __restrict__ colcnt, int vt,
                                                      int* __restrict__ colorder) {
  for (int i = threadIdx.x; i < tt + vt; i += blockDim.x) {
    const bool row = i < tt;
    const int* cnt = row ? rowcnt : colcnt;
    const int n = row ? tt : vt, k = row ? i : i - tt;
    const int ck = cnt[k];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const int cj = cnt[j];
      rank += (cj > ck || (cj == ck && j < k)) ? 1 : 0;
    }
    (row ? roworder : colorder)[rank] = k;
  }
}

// dX rows of one block from the split partials: out (=|+=) sum over z of
// part[z], in split order.  rows x cols fp32, cols a multiple of 4, row
// pitch ldo for out and cols for the partials.
__global__ __launch_bounds__(256) void k_dx_reduce(const float* __restrict__ part, int splits,
                                                   int64_t split_stride, float* __restrict__ out,
                                                   int64_t ldo, int rows, int cols,
                                                   int accumulate) {
  const int64_t nvec = static_cast<int64_t>(rows) * (cols / 4);
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < nvec;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / (cols / 4), c = (i % (cols / 4)) * 4;
    floatx4 s = *reinterpret_cast<const floatx4*>(part + r * cols + c);
    for (int z = 1; z < splits; ++z)
      s += *reinterpret_cast<const floatx4*>(part + z * split_stride + r * cols + c);
    floatx4* o = reinterpret_cast<floatx4*>(out + r * ldo + c);
    if (accumulate) s = *o + s;
    *o = s;
  }
}

// ------------------------------------------- loss on given logits
// The pages' "Trick 1" path ("Fused cross-entropy -- the memory kernel",
// logit-space memory table: probs and dlogits reuse the logits buffer): for
// logits Z the caller holds, one workgroup per row computes
// LSE = m + log sum exp(z - m), the loss term and, if asked, dZ, written
// over Z or into another buffer.  HBM-bound: pass 1 reads the row for
// (reference max, sum-exp, sum z), pass 2 writes dZ.  A row of up to 131072
// bf16 columns stays on chip between the passes; of a longer one, the part
// that fits in LDS.
constexpr int kCeThreads = 1024;
constexpr int kCeUnroll = 4;  // 16-byte loads in flight per thread
// Pass 1 also keeps a row's first kCeCache vectors in LDS (158 KiB of the
// 160 KiB), so pass 2 reads only the rest from memory again: 62% of a
// 128256-column bf16 row.
constexpr int kCeCache = 10112;
// Rows of at most kCeResidentVecs vectors (bf16: 131072 columns) stay on chip
// whole between the passes: thread t's vectors t + 1024 i sit in LDS for
// i < kCeLdsIters (144 KiB) and in registers for the next kCeRegIters (28
// VGPRs), so pass 2 reads no memory.
constexpr int kCeLdsIters = 9, kCeRegIters = 7;
constexpr int kCeResidentVecs = (kCeLdsIters + kCeRegIters) * kCeThreads;
// How far a vector's maximum may pass a thread's reference point m before
// m moves (natural-log units): terms exp(z - m) stay below e^16 = 2^23.1, so
// a thread's sum of up to 2^21 of them cannot overflow.
constexpr float kCeLag = 16.0f;

template <typename T>
struct CeVec;
template <>
struct CeVec<bf16> {
  static constexpr int E = 8;  // elements per 16-byte vector
  __device__ __forceinline__ static void unpack(const u32x4& r, float (&f)[E]) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = static_cast<float>(v[e]);
  }
  __device__ __forceinline__ static u32x4 pack(const float (&f)[E]) {  // round to nearest even
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 h = {static_cast<bf16>(f[2 * i]), static_cast<bf16>(f[2 * i + 1])};
      r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
  }
};
template <>
struct CeVec<float> {
  static constexpr int E = 4;
  __device__ __forceinline__ static void unpack(const u32x4& r, float (&f)[E]) {
    const floatx4 v = __builtin_bit_cast(floatx4, r);  // (whole-vector cast)
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = v[i];
  }
  __device__ __forceinline__ static u32x4 pack(const float (&f)[E]) {
    const floatx4 v = {f[0], f[1], f[2], f[3]};
    return __builtin_bit_cast(u32x4, v);
  }
};

struct CeArgs {
  const void* Z;
  int64_t ldz;  // elements
  void* dZ;     // may equal Z; NULL: no gradient
  int64_t lddz;
  const int32_t* labels;
  int N, V, ignore, reduction;  // reduction: 0 mean, 1 sum, 2 none
  float eps, zloss;
  const float* grad;  // per-token upstream gradient (none), or NULL
  const Ctrl* ctrl;   // scale_bwd = g / D (mean, sum)
  float* lse;
  float* rowloss;  // per-row loss terms
  // GIVEN with fp32 logits: the forward's split row statistics (m, log2 l)
  // of each row, or NULL (then m = LSE, log2 l = 0)
  const float2* stat;
};

// NC: vectors of the row kept in LDS between the passes (0: none, for the
// loss alone, whose workgroups then overlap at row boundaries).  RC > 0: the
// whole row stays on chip (NC = kCeLdsIters x kCeThreads vectors in LDS, RC
// per thread in registers; the row has at most NC + RC x kCeThreads vectors)
// and both passes walk it with compile-time indices.
// GIVEN: lse holds each valid row's LSE already (the store-logits variant,
// whose forward computed it from the fp32 accumulators); only pass 2 runs,
// neither lse nor the loss terms are written, and dZ leaves out the scale
// g / D, which the gradient products apply in fp32 (the per-token g_i of
// reduction none is kept).
template <typename T, bool GIVEN, int NC, int RC = 0>
__global__ __launch_bounds__(kCeThreads) void k_ce_logits(CeArgs a) {
  static_assert(RC == 0 || (!GIVEN && NC % kCeThreads == 0), "resident rows: LDS whole iterations");
  typedef CeVec<T> CV;
  constexpr int E = CV::E;
  __shared__ floatx4 s_part[kCeThreads / 64];
  __shared__ float s_bcast[2];
  __shared__ u32x4 s_cache[NC > 0 ? NC : 1];  // the row's first vectors (pass 1 -> 2)
  u32x4 rcache[RC > 0 ? RC : 1];               // RC > 0: the rest of the row
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int y = a.labels[row];
  const bool valid = label_ok(y, a.ignore, a.V);
  const int nv = (a.V + E - 1) / E;  // 16-byte vectors per row
  const int nvf = a.V / E;           // whole vectors of the row
  const T* zrow = static_cast<const T*>(a.Z) + row * a.ldz;
  T* drow = a.dZ ? static_cast<T*>(a.dZ) + row * a.lddz : nullptr;
  // Loads past the row's vectors return zeros and stores there are dropped:
  // the descriptors cover exactly the row's nv vectors.
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(zrow, static_cast<int64_t>(nv) * 16);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(drow, drow ? static_cast<int64_t>(nv) * 16 : 0);
  // Elements past V (only in vector nv-1, or in whole vectors past the row)
  // become -inf for the max and the exponentials, are left out of the logit
  // sum, and get a dZ of 0.
  auto pad = [](float (&f)[E], int lim, float v) {
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = (e < lim) ? f[e] : v;
  };
  if (!valid) {  // ignored (or invalid) label: no loss, zero gradient row
    if (!GIVEN && tid == 0) {
      a.lse[row] = NAN;
      a.rowloss[row] = (y == a.ignore || a.reduction != 2) ? 0.0f : NAN;
    }
    if (drow)
      for (int j = tid; j < nv; j += kCeThreads)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, rd, j * 16, 0, 0);
    return;
  }

  // LSE = m + lg ln 2, with the row's reference m (its maximum, or at most
  // kCeLag below it) and lg = log2 of the sum of exp(z - m) kept apart for
  // the exponents of pass 2 (fp32)
  float L, m_row, lg_row;
  if constexpr (GIVEN) {
    L = a.lse[row];
    const float2 sv = a.stat ? a.stat[row] : float2{L, 0.0f};
    m_row = sv.x;
    lg_row = sv.y;
  } else {
    // pass 1: running (m, sum-exp, sum z) of this thread's vectors.  m is a
    // reference point for the exponentials, not the running maximum: it moves
    // up to a vector's maximum only when that passes it by more than kCeLag,
    // so a term exp(z - m) stays below e^kCeLag and most vectors need no
    // rescaling of the sum.  The sum then stands for sum exp(z - m) at that m,
    // which is what the merges and LSE = m + log sum take.
    // Before the first vector with a finite maximum the terms use a
    // reference of +inf, so that they vanish instead of forming inf - inf.
    float m = -INFINITY, mt = INFINITY, mtl = INFINITY, mup = -INFINITY, l = 0.0f, zs = 0.0f;
    const bool smooth = a.eps != 0.0f;
    // WHOLE (workgroup-uniform): every thread's vector of this iteration lies
    // inside the row's whole vectors, so no element needs a tail mask
    auto accumulate = [&](const u32x4& rv, int j, bool whole) {
      float f[E];
      CV::unpack(rv, f);
      if (whole) {
        if (smooth) {
#pragma unroll
          for (int e = 0; e < E; ++e) zs += f[e];
        }
      } else {
        const int lim = a.V - j * E;
        if (smooth) {
#pragma unroll
          for (int e = 0; e < E; ++e) zs += (e < lim) ? f[e] : 0.0f;
        }
        pad(f, lim, -INFINITY);
      }
      float vm = f[0];
#pragma unroll
      for (int e = 1; e < E; ++e) vm = fmaxf(vm, f[e]);
      if (vm > mup) {  // first finite maximum, or one far above the reference
        l = (m == -INFINITY) ? 0.0f : l * hw_exp2((m - vm) * kLog2e);
        m = mt = vm;
        mtl = vm * kLog2e;
        mup = vm + kCeLag;
      }
      // fp32: exp2((z - m) log2e), within kCeLag of exact at any |m| (the
      // one-FMA form carries an error of |m| 2^-25 into every term)
      auto term = [&](float z) {
        return hw_exp2((sizeof(T) == 4) ? (z - mt) * kLog2e : fmaf(z, kLog2e, -mtl));
      };
      float acc = term(f[0]);
#pragma unroll
      for (int e = 1; e < E; ++e) acc += term(f[e]);
      l += acc;
    };
    if constexpr (RC > 0) {
      // the whole row: vectors past the row load as zero and are padded out
#pragma unroll
      for (int g = 0; g < NC / kCeThreads + RC; g += kCeUnroll) {
        u32x4 r[kCeUnroll];
#pragma unroll
        for (int u = 0; u < kCeUnroll; ++u)
          if (g + u < NC / kCeThreads + RC) r[u] = buf_load16(rz, (tid + (g + u) * kCeThreads) * 16);
#pragma unroll
        for (int u = 0; u < kCeUnroll; ++u) {
          const int i = g + u;
          if (i >= NC / kCeThreads + RC) break;
          if (i < NC / kCeThreads)
            s_cache[tid + i * kCeThreads] = r[u];
          else
            rcache[i - NC / kCeThreads] = r[u];
          accumulate(r[u], tid + i * kCeThreads, (i + 1) * kCeThreads <= nvf);
        }
      }
    } else {
      for (int j0 = tid; j0 < nv; j0 += kCeUnroll * kCeThreads) {
        u32x4 r[kCeUnroll];
#pragma unroll
        for (int u = 0; u < kCeUnroll; ++u) r[u] = buf_load16(rz, (j0 + u * kCeThreads) * 16);
#pragma unroll
        for (int u = 0; u < kCeUnroll; ++u) {
          if (j0 + u * kCeThreads < NC) s_cache[j0 + u * kCeThreads] = r[u];
          accumulate(r[u], j0 + u * kCeThreads, j0 - tid + (u + 1) * kCeThreads <= nvf);
        }
      }
    }
    // wave, then fixed-order workgroup merge of (m, l, sum z)
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) {
      float t0 = 0.0f;
      const float m2 = __shfl_xor(m, sh), l2 = __shfl_xor(l, sh), z2 = __shfl_xor(zs, sh);
      lse_merge(m, l, t0, zs, m2, l2, 0.0f, z2);
    }
    if (lane == 0) s_part[wave] = floatx4{m, l, 0.0f, zs};
    __syncthreads();
    if (tid == 0) {
      floatx4 st = s_part[0];
      for (int w = 1; w < kCeThreads / 64; ++w) lse_merge(st, s_part[w]);
      const float lg = hw_log2(st[1]);
      const float Lr = st[0] + lg * kLn2;
      const float zy = static_cast<float>(zrow[y]);  // the target logit
      // (m - z_y) first: exact when the target logit is near the max
      float term = (st[0] - (1.0f - a.eps) * zy) + lg * kLn2;
      if (smooth) term -= (a.eps / static_cast<float>(a.V)) * st[3];
      if (a.zloss != 0.0f) term += a.zloss * Lr * Lr;
      a.lse[row] = Lr;
      a.rowloss[row] = term;
      s_bcast[0] = st[0];
      s_bcast[1] = lg;
    }
    if (!drow) return;
    __syncthreads();
    m_row = s_bcast[0];
    lg_row = s_bcast[1];
    L = m_row + lg_row * kLn2;
  }

  // pass 2: dZ = (p (1 + 2 alpha L) - eps/V - (1-eps)[i = y]) * scale, p = exp(z - L)
  const float scale = (a.reduction == 2) ? (a.grad ? a.grad[row] : 1.0f)
                                         : (GIVEN ? 1.0f : a.ctrl->scale_bwd);
  const float ga = (1.0f + 2.0f * a.zloss * L) * scale;
  const float gb = (a.eps / static_cast<float>(a.V)) * scale;
  const float gy = (1.0f - a.eps) * scale;
  const float Ll = L * kLog2e;
  const int jy = y / E, ey = y % E;
  // dZ over Z: streaming stores (the lines were just read and are not read
  // again); into another buffer the default policy measured faster
  const bool inplace = a.dZ == a.Z;
  // One vector j.  PLAIN (workgroup-uniform): the iteration holds neither
  // the label's vector nor one past the row's whole vectors, so it needs no
  // one-hot term and no tail mask.
  auto emit = [&](const u32x4& rv, int j, int first) {
    float f[E];
    CV::unpack(rv, f);
    // fp32: exp2((z - m) log2e - log2 l), exact near the max at any |LSE|;
    // bf16 logits carry far coarser rounding and keep the one-FMA form
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = (sizeof(T) == 4) ? fmaf(f[e] - m_row, kLog2e, -lg_row)
                                       : fmaf(f[e], kLog2e, -Ll);
      f[e] = fmaf(hw_exp2(x), ga, -gb);
    }
    const bool plain = first + kCeThreads <= nvf && (jy < first || jy >= first + kCeThreads);
    if (!plain) {
      if (j == jy) {  // the one lane holding the label
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] -= (e == ey) ? gy : 0.0f;
      }
      const int lim = a.V - j * E;
      if (lim < E) pad(f, lim, 0.0f);
    }
    const u32x4 out = CV::pack(f);
    if (inplace)
      __builtin_amdgcn_raw_buffer_store_b128(out, rd, j * 16, 0, kBufNonTemporal);
    else
      __builtin_amdgcn_raw_buffer_store_b128(out, rd, j * 16, 0, 0);
  };
  if constexpr (RC > 0) {
    // from LDS and registers only; stores past the row are dropped
#pragma unroll
    for (int i = 0; i < NC / kCeThreads + RC; ++i)
      emit(i < NC / kCeThreads ? s_cache[tid + i * kCeThreads] : rcache[i - NC / kCeThreads],
           tid + i * kCeThreads, i * kCeThreads);
  } else {
    for (int j0 = tid; j0 < nv; j0 += kCeUnroll * kCeThreads) {
      u32x4 r[kCeUnroll];
#pragma unroll
      for (int u = 0; u < kCeUnroll; ++u) {
        const int j = j0 + u * kCeThreads;
        r[u] = (j < NC) ? s_cache[j] : buf_load16(rz, j * 16);
      }
#pragma unroll
      for (int u = 0; u < kCeUnroll; ++u)
        emit(r[u], j0 + u * kCeThreads, j0 - tid + u * kCeThreads);
    }
  }
}

// ------------------------------------------------------------- launching
template <typename T>
struct ShapeOf;
template <>
struct ShapeOf<bf16> {
  typedef Cfg<ShapeBf16, bf16> C;
};
template <>
struct ShapeOf<float> {
  typedef Cfg<ShapeF32, float> C;
};

int cdiv_i(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

#define FCE_CHECK_LAUNCH()                      \
  do {                                          \
    hipError_t e_ = hipGetLastError();          \
    if (e_ != hipSuccess) return e_;            \
  } while (0)

template <typename T>
hipError_t run_forward(const Plan& p, const T* X, const T* W, const int32_t* labels,
                       const LossOpts& o, float* loss, float* lse, char* ws, hipStream_t st,
                       KernelTimer* timer) {
  const int ignore = o.ignore;
  const float eps = o.eps;
  const bool none = o.reduction == Reduction::None;
  typedef typename ShapeOf<T>::C C;
  Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + p.off_ctrl);
  float* blockloss = reinterpret_cast<float*>(ws + p.off_blockloss);
  floatx4* part = reinterpret_cast<floatx4*>(ws + p.off_part);
  float2* stat = p.stat_bytes ? reinterpret_cast<float2*>(ws + p.off_stat) : nullptr;
  const int N = static_cast<int>(p.N), H = static_cast<int>(p.H), V = static_cast<int>(p.V);
  if (N > 0) {
    FwdArgs<T> fa{X, W, labels, N, H, V, ignore,
                  static_cast<int>(p.fwd_tok_tiles), static_cast<int>(p.fwd_voc_tiles),
                  static_cast<int>(p.fwd_splits), 1, p.n_pad, part};
    // one XCD (32 CUs) covers gm token tiles x all splits
    fa.group_m = static_cast<int>(std::max<int64_t>(1, 32 / std::max<int64_t>(p.fwd_splits, 1)));
    const int grid = fa.tok_tiles * fa.splits;
    const double flops = 2.0 * static_cast<double>(p.N) * p.V * p.H;
    timer->begin("fwd_lse", flops, st);
    if (eps != 0.0f)
      launch_fwd_lse<C, true, false>(fa, grid, st);
    else
      launch_fwd_lse<C, false, false>(fa, grid, st);
    FCE_CHECK_LAUNCH();
    timer->end(st);
    timer->begin("lse_merge", 0.0, st);
    k_lse_merge<<<cdiv_i(N, kLossBlock), kLossBlock, 0, st>>>(
        part, fa.splits, p.n_pad, labels, N, V, ignore, eps, o.zloss, lse, blockloss,
        none ? loss : nullptr, stat);
    FCE_CHECK_LAUNCH();
    timer->end(st);
  }
  if (none) return hipSuccess;  // the per-token losses are the output
  timer->begin("loss_final", 0.0, st);
  k_loss_final<<<1, 256, 0, st>>>(blockloss, N > 0 ? static_cast<int>(p.n_loss_blocks) : 0, ctrl,
                                  loss);
  FCE_CHECK_LAUNCH();
  timer->end(st);
  return hipSuccess;
}

// Kept-block lists of one logit block (filtered products).
struct FilterLists {
  const int* rowlist;  // [tt][vt]: per token tile, kept vocabulary tiles
  const int* rowcnt;
  const int* roworder;  // token tiles by descending kept count
  const int* collist;  // [vt][tt]: per vocabulary tile, kept token tiles
  const int* colcnt;
  const int* colorder;  // vocabulary tiles by descending kept count
  int tt, vt;
};

// The two gradient products of one logit block: dZ is [ntok][>= nvoc
// rounded up to the tile] at dz with row pitch ldz, for tokens tok0.. and
// vocabulary columns voc0...  acc_dw / acc_dx: add to the previous block's
// values instead of storing.  dxpart: the plan's dx_splits partials of dX
// ([splits][ntok][H] fp32) when it splits the dX product.
template <typename T>
hipError_t grad_products(const Plan& p, const T* X, const T* W, const T* dz, int64_t ldz,
                         int64_t tok0, int ntok, int64_t voc0, int nvoc, bool acc_dw, bool acc_dx,
                         const Ctrl* ctrl, const int32_t* flag, float* dX, float* dW,
                         float* dxpart, const FilterLists* fl, const T* Xt, int64_t ldxt,
                         hipStream_t st, KernelTimer* timer, const char* name_dw,
                         const char* name_dx, const char* name_pair) {
  typedef typename ShapeOf<T>::C C;
  const int64_t H = p.H;
  const int h_tiles = cdiv_i(H, C::BN);
  const int tok_tiles = cdiv_i(ntok, C::BN);
  const int voc_tiles = cdiv_i(nvoc, C::BM);
  const int nvoc_cov = voc_tiles * C::BM;
  const double blk_flops = 2.0 * static_cast<double>(ntok) * nvoc * H;

  // dW[voc0 : voc0+nvoc] (=|+=) s * dZ^T X[tok0 : tok0+ntok]
  GradArgs<T> gw;
  gw.A = Opnd<T>{dz, ldz, nvoc, ntok};                            // (v, t) at dz[t*ldz + v]
  gw.B = Opnd<T>{X + tok0 * H, H, static_cast<int>(H), ntok};    // (h, t) at X[t*H + h]
  gw.K = ntok;
  gw.m_valid = nvoc;
  gw.n_valid = static_cast<int>(H);
  gw.tm_tiles = voc_tiles;
  gw.tn_tiles = h_tiles;
  gw.group_m = 2;
  gw.out = dW + voc0 * H;
  gw.ldo = H;
  gw.ctrl = ctrl;
  gw.accumulate = acc_dw;
  gw.flag = flag;
  gw.ksplit = ntok;
  gw.split_stride = 0;
  gw.klist = fl ? fl->collist : nullptr;
  gw.kcount = fl ? fl->colcnt : nullptr;
  gw.list_ld = fl ? fl->tt : 0;
  gw.korder = fl ? fl->colorder : nullptr;
  // With X^T at hand (bf16, unfiltered): (dW)^T = X^T dZ, whose A operand
  // (X^T, rows h) is K-major, so the product takes the ping-pong K loop of
  // the dX product; the tile is written transposed.  K runs over the token
  // tiles: X^T is zero past N and dZ^T rows past the block's tokens load as
  // zero, so the extra columns add nothing.
  GradArgs<T> gt = gw;
  if (Xt != nullptr) {
    gt.A = Opnd<T>{Xt + tok0, ldxt, static_cast<int>(H), tok_tiles * C::BN};  // (h, t) at Xt[h*ldxt + t]
    gt.B = Opnd<T>{dz, ldz, nvoc, ntok};                                      // (v, t) at dz[t*ldz + v]
    gt.K = tok_tiles * C::BN;
    gt.m_valid = static_cast<int>(H);
    gt.n_valid = nvoc;
    gt.tm_tiles = h_tiles;
    gt.tn_tiles = voc_tiles;
    gt.ksplit = gt.K;
    // groups of 4 H-tile rows: a squarer patch of tiles per XCD than the 2
    // vocabulary rows of dZ^T X (6.48 against 6.56 ms at 8192 x 4096 x 12288)
    gt.group_m = 4;
  }
  // dX[tok0 : tok0+ntok] (=|+=) s * dZ W[voc0 : voc0+nvoc]
  GradArgs<T> gx;
  gx.A = Opnd<T>{dz, ldz, ntok, nvoc_cov};                         // (t, v) at dz[t*ldz + v]
  gx.B = Opnd<T>{W + voc0 * H, H, static_cast<int>(H), nvoc};     // (h, v) at W[v*H + h]
  gx.K = nvoc_cov;
  gx.m_valid = ntok;
  gx.n_valid = static_cast<int>(H);
  gx.tm_tiles = tok_tiles;
  gx.tn_tiles = h_tiles;
  gx.group_m = 2;
  gx.out = dX + tok0 * H;
  gx.ldo = H;
  gx.ctrl = ctrl;
  gx.accumulate = acc_dx;
  gx.flag = flag;
  gx.ksplit = nvoc_cov;
  gx.split_stride = 0;
  gx.klist = fl ? fl->rowlist : nullptr;
  gx.kcount = fl ? fl->rowcnt : nullptr;
  gx.list_ld = fl ? fl->vt : 0;
  gx.korder = fl ? fl->roworder : nullptr;
  // split over the vocabulary when the plan asks for it: whole tiles per split
  const int ksplit = cdiv_i(cdiv_i(nvoc_cov, static_cast<int>(p.dx_splits)), C::BM) * C::BM;
  const int splits = fl ? 1 : cdiv_i(nvoc_cov, ksplit);
  if (splits > 1) {
    gx.ksplit = ksplit;
    gx.out = dxpart;
    gx.accumulate = 0;
    gx.split_stride = static_cast<int64_t>(ntok) * H;
  }
  const int n_dw = voc_tiles * h_tiles, n_dx = tok_tiles * h_tiles;
  if constexpr (sizeof(T) == 2) {
    if (fl != nullptr) {
      // the filtered products in one launch
      const int dx_first = nvoc_cov > gw.K;
      timer->begin(name_pair, 2.0 * blk_flops, st);
      k_bwd_grad_pair_filt<C><<<n_dw + n_dx, C::NT, 0, st>>>(gw, gt, gx, n_dw, n_dx, dx_first,
                                                             Xt != nullptr);
      FCE_CHECK_LAUNCH();
      timer->end(st);
    } else {
      // one launch for both products (bf16, unfiltered); the tiles with the
      // longer contraction first
      const int dx_first = (splits > 1 ? ksplit : nvoc_cov) > (Xt != nullptr ? gt.K : gw.K);
      timer->begin(name_pair, 2.0 * blk_flops, st);
      if (Xt != nullptr)
        k_bwd_grad_pair<C, true, true><<<n_dw + n_dx * splits, C::NT, 0, st>>>(gt, gx, n_dw, n_dx,
                                                                               splits, dx_first);
      else
        k_bwd_grad_pair<C, false, false><<<n_dw + n_dx * splits, C::NT, 0, st>>>(
            gw, gx, n_dw, n_dx, splits, dx_first);
      FCE_CHECK_LAUNCH();
      timer->end(st);
    }
  }
  if constexpr (sizeof(T) == 4) {  // fp32: one launch per product
    timer->begin(name_dw, blk_flops, st);
    k_bwd_grad<C, false, false><<<n_dw, C::NT, 0, st>>>(gw);
    FCE_CHECK_LAUNCH();
    timer->end(st);
    timer->begin(name_dx, blk_flops, st);
    k_bwd_grad<C, true, false><<<dim3(n_dx, splits), C::NT, 0, st>>>(gx);
    FCE_CHECK_LAUNCH();
    timer->end(st);
  }
  if (splits > 1) {
    timer->begin("dx_reduce", 0.0, st);
    k_dx_reduce<<<1024, 256, 0, st>>>(dxpart, splits, gx.split_stride, dX + tok0 * H, H, ntok,
                                      static_cast<int>(H), acc_dx);
    FCE_CHECK_LAUNCH();
    timer->end(st);
  }
  return hipSuccess;
}

// Writes X^T into the workspace for the dW products and points *xt at it,
// when the plan has room for it (bf16); *xt = nullptr otherwise.
template <typename T>
hipError_t transpose_x(const Plan& p, const T* X, char* ws, hipStream_t st, KernelTimer* timer,
                       const T** xt) {
  *xt = nullptr;
  if constexpr (sizeof(T) == 2) {
    if (p.xt_bytes > 0) {
      T* out = reinterpret_cast<T*>(ws + p.off_xt);
      timer->begin("x_transpose", 0.0, st);
      k_transpose_x<<<dim3(static_cast<unsigned>(cdiv_i(p.ldxt, 64)),
                           static_cast<unsigned>(cdiv_i(p.H, 64))),
                      256, 0, st>>>(X, static_cast<int>(p.N), static_cast<int>(p.H), out, p.ldxt);
      FCE_CHECK_LAUNCH();
      timer->end(st);
      *xt = out;
    }
  }
  return hipSuccess;
}

template <typename T>
hipError_t run_backward(const Plan& p, const T* X, const T* W, const int32_t* labels,
                        const LossOpts& o, const float* lse, const float2* stat,
                        const float* grad_tok, float* dX, float* dW, char* ws, hipStream_t st,
                        KernelTimer* timer) {
  const int ignore = o.ignore;
  const float eps = o.eps;
  typedef typename ShapeOf<T>::C C;
  const Ctrl* ctrl = reinterpret_cast<const Ctrl*>(ws + p.off_ctrl);
  const int32_t* flags = reinterpret_cast<const int32_t*>(ws + p.off_flags);
  T* dz = reinterpret_cast<T*>(ws + p.off_scratch);
  float* dxpart = reinterpret_cast<float*>(ws + p.off_dxpart);
  const int64_t N = p.N, H = p.H, V = p.V;
  const bool filt = sizeof(T) == 2 && p.variant == Variant::Filtered;
  uint8_t* keep = reinterpret_cast<uint8_t*>(ws + p.off_keep);
  unsigned long long* fstats = reinterpret_cast<unsigned long long*>(ws + p.off_ctrl +
                                                                     kOffFilterStats);
  if (filt) {  // kept / all tile counters of this call, and every block's kept flags
    timer->begin("fill_zero", 0.0, st);
    k_fill_zero<<<1, 256, 0, st>>>(reinterpret_cast<float*>(fstats), 4);
    FCE_CHECK_LAUNCH();
    const int64_t nk = static_cast<int64_t>((p.keep_bytes + 3) / 4);  // within the 256-byte padding
    k_fill_zero<<<static_cast<int>(std::min<int64_t>(1024, std::max<int64_t>(1, (nk + 255) / 256))),
                  256, 0, st>>>(reinterpret_cast<float*>(keep), nk);
    FCE_CHECK_LAUNCH();
    timer->end(st);
  }
  if (N == 0) {
    timer->begin("fill_zero", 0.0, st);
    k_fill_zero<<<1024, 256, 0, st>>>(dW, V * H);
    FCE_CHECK_LAUNCH();
    timer->end(st);
    return hipSuccess;
  }
  // X^T for the dW products (when the plan has room for it)
  const T* xt = nullptr;
  {
    const hipError_t e = transpose_x(p, X, ws, st, timer, &xt);
    if (e != hipSuccess) return e;
  }
  for (int64_t ia = 0; ia < p.a; ++ia) {
    const int64_t tok0 = ia * p.CN;
    const int ntok = static_cast<int>(std::min(p.CN, N - tok0));
    const int tok_tiles = cdiv_i(ntok, C::BN);
    for (int64_t ib = 0; ib < p.b; ++ib) {
      const int64_t voc0 = ib * p.CV;
      const int nvoc = static_cast<int>(std::min(p.CV, V - voc0));
      const int voc_tiles = cdiv_i(nvoc, C::BM);
      const double blk_flops = 2.0 * static_cast<double>(ntok) * nvoc * H;

      uint8_t* const keep_blk = filt ? keep + (ia * p.b + ib) * p.filt_tt * p.filt_vt : nullptr;
      DzArgs<T> da{X + tok0 * H, W + voc0 * H, labels + tok0, lse + tok0, ntok, nvoc,
                   static_cast<int>(voc0), static_cast<int>(H), static_cast<int>(V), ignore, eps,
                   o.zloss, grad_tok ? grad_tok + tok0 : nullptr, voc_tiles, tok_tiles, 4, dz,
                   p.ldz, flags + ia, keep_blk, stat ? stat + tok0 : nullptr};
      // bf16 with H % 128 == 0: about one workgroup per CU, each streaming a
      // run of vocabulary tiles
      const bool dz_stream = sizeof(T) == 2 && H % 128 == 0 && H >= 256;
      timer->begin("bwd_dz", blk_flops, st);
      if constexpr (sizeof(T) == 2) {
        if (filt && dz_stream) {
          // the dZ stream with the filter votes (flags zeroed at the start)
          const int splits = std::max(1, std::min(voc_tiles, kNumCUs / tok_tiles));
          da.group_m = std::max(1, 32 / splits);
          k_bwd_dz_stream<C, true><<<tok_tiles * splits, C::NT, 0, st>>>(da, splits);
        } else if (filt) {
          if (H % 32 == 0)
            k_bwd_dz<C, true, true><<<voc_tiles * tok_tiles, C::NT, 0, st>>>(da);
          else
            k_bwd_dz<C, false, true><<<voc_tiles * tok_tiles, C::NT, 0, st>>>(da);
        } else if (dz_stream) {
          const int splits = std::max(1, std::min(voc_tiles, kNumCUs / tok_tiles));
          da.group_m = std::max(1, 32 / splits);
          k_bwd_dz_stream<C><<<tok_tiles * splits, C::NT, 0, st>>>(da, splits);
        } else if (H % 32 == 0) {
          k_bwd_dz<C, true, false><<<voc_tiles * tok_tiles, C::NT, 0, st>>>(da);
        } else {
          k_bwd_dz<C, false, false><<<voc_tiles * tok_tiles, C::NT, 0, st>>>(da);
        }
      } else {
        if (H % 32 == 0)
          k_bwd_dz<C, true, false><<<voc_tiles * tok_tiles, C::NT, 0, st>>>(da);
        else
          k_bwd_dz<C, false, false><<<voc_tiles * tok_tiles, C::NT, 0, st>>>(da);
      }
      FCE_CHECK_LAUNCH();
      timer->end(st);

      FilterLists fl{reinterpret_cast<const int*>(ws + p.off_rowlist),
                     reinterpret_cast<const int*>(ws + p.off_rowcnt),
                     reinterpret_cast<const int*>(ws + p.off_roworder),
                     reinterpret_cast<const int*>(ws + p.off_collist),
                     reinterpret_cast<const int*>(ws + p.off_colcnt),
                     reinterpret_cast<const int*>(ws + p.off_colorder), tok_tiles, voc_tiles};
      if (filt) {
        timer->begin("filter_lists", 0.0, st);
        k_filter_lists<<<tok_tiles + voc_tiles, 64, 0, st>>>(
            keep_blk, tok_tiles, voc_tiles, reinterpret_cast<int*>(ws + p.off_rowlist),
            reinterpret_cast<int*>(ws + p.off_rowcnt), reinterpret_cast<int*>(ws + p.off_collist),
            reinterpret_cast<int*>(ws + p.off_colcnt), fstats);
        FCE_CHECK_LAUNCH();
        k_filter_order<<<1, 256, 0, st>>>(
            reinterpret_cast<const int*>(ws + p.off_rowcnt), tok_tiles,
            reinterpret_cast<int*>(ws + p.off_roworder),
            reinterpret_cast<const int*>(ws + p.off_colcnt), voc_tiles,
            reinterpret_cast<int*>(ws + p.off_colorder));
        FCE_CHECK_LAUNCH();
        timer->end(st);
      }
      const hipError_t e = grad_products<T>(p, X, W, dz, p.ldz, tok0, ntok, voc0, nvoc, ia > 0,
                                            ib > 0, ctrl, flags + ia, dX, dW, dxpart,
                                            filt ? &fl : nullptr, xt, p.ldxt, st, timer, "bwd_dw",
                                            "bwd_dx", "bwd_grad");
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Store-logits fused forward and backward (the Liger-style design of
// "Chunked and Fused Cross-Entropy", llms.blog, "LinkedIn Liger Kernel": a
// token chunk's logits are kept and overwritten in place by their gradient).
// Per block of C_N tokens: the forward keeps the block's logits [C_N][V] in
// the workspace while it reduces them to LSE partials; the merge gives LSE and
// the loss terms; a streaming pass turns the logits into dZ in place; then
// the two gradient products.  Executed work is 6NVH (no recompute).
template <typename T>
hipError_t run_fused_store(const Plan& p, const T* X, const T* W, const int32_t* labels,
                           const LossOpts& o, float* loss, float* lse, float* dX, float* dW,
                           char* ws, hipStream_t st, KernelTimer* timer) {
  typedef typename ShapeOf<T>::C C;
  const bool none = o.reduction == Reduction::None;
  Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + p.off_ctrl);
  const int32_t* flags = reinterpret_cast<const int32_t*>(ws + p.off_flags);
  float* blockloss = reinterpret_cast<float*>(ws + p.off_blockloss);
  floatx4* part = reinterpret_cast<floatx4*>(ws + p.off_part);
  T* zs = reinterpret_cast<T*>(ws + p.off_scratch);
  float* dxpart = reinterpret_cast<float*>(ws + p.off_dxpart);
  float2* stat = p.stat_bytes ? reinterpret_cast<float2*>(ws + p.off_stat) : nullptr;
  const int64_t N = p.N, H = p.H, V = p.V;
  if (N == 0) {
    timer->begin("fill_zero", 0.0, st);
    k_fill_zero<<<1024, 256, 0, st>>>(dW, V * H);
    FCE_CHECK_LAUNCH();
    timer->end(st);
  }
  const T* xt = nullptr;
  if (N > 0) {
    const hipError_t e = transpose_x(p, X, ws, st, timer, &xt);
    if (e != hipSuccess) return e;
  }
  for (int64_t ia = 0; ia < p.a; ++ia) {
    const int64_t tok0 = ia * p.CN;  // a multiple of kLossBlock
    const int ntok = static_cast<int>(std::min(p.CN, N - tok0));
    FwdArgs<T> fa{X + tok0 * H, W, labels + tok0, ntok, static_cast<int>(H), static_cast<int>(V),
                  o.ignore, cdiv_i(ntok, C::BN), static_cast<int>(p.fwd_voc_tiles),
                  static_cast<int>(p.fwd_splits), 1, p.n_pad, part, zs, p.ldz};
    fa.group_m = static_cast<int>(std::max<int64_t>(1, 32 / std::max<int64_t>(p.fwd_splits, 1)));
    const double blk_flops = 2.0 * static_cast<double>(ntok) * V * H;
    timer->begin("sl_fwd", blk_flops, st);
    if (o.eps != 0.0f)
      launch_fwd_lse<C, true, true>(fa, fa.tok_tiles * fa.splits, st);
    else
      launch_fwd_lse<C, false, true>(fa, fa.tok_tiles * fa.splits, st);
    FCE_CHECK_LAUNCH();
    timer->end(st);
    timer->begin("lse_merge", 0.0, st);
    k_lse_merge<<<cdiv_i(ntok, kLossBlock), kLossBlock, 0, st>>>(
        part, fa.splits, p.n_pad, labels + tok0, ntok, static_cast<int>(V), o.ignore, o.eps,
        o.zloss, lse + tok0, blockloss + tok0 / kLossBlock, none ? loss + tok0 : nullptr,
        stat ? stat + tok0 : nullptr);
    FCE_CHECK_LAUNCH();
    timer->end(st);
    // logits -> dZ in place (upstream gradient 1 per token for reduction none)
    CeArgs ca{zs, p.ldz, zs, p.ldz, labels + tok0, ntok, static_cast<int>(V), o.ignore,
              static_cast<int>(o.reduction), o.eps, o.zloss, nullptr, ctrl, lse + tok0, nullptr,
              stat ? stat + tok0 : nullptr};
    timer->begin("sl_dz", 0.0, st);
    k_ce_logits<T, true, 0><<<ntok, kCeThreads, 0, st>>>(ca);
    FCE_CHECK_LAUNCH();
    timer->end(st);
    const hipError_t e = grad_products<T>(p, X, W, zs, p.ldz, tok0, ntok, 0, static_cast<int>(V),
                                          ia > 0, false, ctrl, flags + ia, dX, dW, dxpart,
                                          nullptr, xt, p.ldxt, st, timer, "sl_dw", "sl_dx",
                                          "sl_grad");
    if (e != hipSuccess) return e;
  }
  if (none) return hipSuccess;
  timer->begin("loss_final", 0.0, st);
  k_loss_final<<<1, 256, 0, st>>>(blockloss, N > 0 ? static_cast<int>(p.n_loss_blocks) : 0, ctrl,
                                  loss);
  FCE_CHECK_LAUNCH();
  timer->end(st);
  return hipSuccess;
}

}  // namespace

hipError_t launch_fused_store(const Plan& p, const void* X, const void* W, const int32_t* labels,
                              const LossOpts& o, float* loss, float* lse, float* dX, float* dW,
                              char* ws, hipStream_t st, KernelTimer* timer) {
  if (p.dtype == Dtype::BF16)
    return run_fused_store<bf16>(p, static_cast<const bf16*>(X), static_cast<const bf16*>(W),
                                 labels, o, loss, lse, dX, dW, ws, st, timer);
  return run_fused_store<float>(p, static_cast<const float*>(X), static_cast<const float*>(W),
                                labels, o, loss, lse, dX, dW, ws, st, timer);
}

hipError_t launch_label_scan(const Plan& p, const int32_t* labels, const LossOpts& o,
                             const float* grad, char* ws, hipStream_t st, KernelTimer* timer) {
  Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + p.off_ctrl);
  int32_t* flags = reinterpret_cast<int32_t*>(ws + p.off_flags);
  timer->begin("label_scan", 0.0, st);
  k_label_scan<<<1, 1024, 0, st>>>(labels, static_cast<int>(p.N), static_cast<int>(p.V), o.ignore,
                                   static_cast<int>(o.reduction), grad, ctrl, flags,
                                   static_cast<int>(p.CN),
                                   static_cast<int>(std::max<int64_t>(p.a, 1)));
  FCE_CHECK_LAUNCH();
  timer->end(st);
  return hipSuccess;
}

hipError_t launch_forward(const Plan& p, const void* X, const void* W, const int32_t* labels,
                          const LossOpts& o, float* loss, float* lse, char* ws, hipStream_t st,
                          KernelTimer* timer) {
  if (p.dtype == Dtype::BF16)
    return run_forward<bf16>(p, static_cast<const bf16*>(X), static_cast<const bf16*>(W), labels,
                             o, loss, lse, ws, st, timer);
  return run_forward<float>(p, static_cast<const float*>(X), static_cast<const float*>(W), labels,
                            o, loss, lse, ws, st, timer);
}

hipError_t launch_backward(const Plan& p, const void* X, const void* W, const int32_t* labels,
                           const LossOpts& o, const float* lse, bool use_stats,
                           const float* grad_tok, float* dX, float* dW, char* ws, hipStream_t st,
                           KernelTimer* timer) {
  const float2* stat = (use_stats && p.stat_bytes)
                           ? reinterpret_cast<const float2*>(ws + p.off_stat)
                           : nullptr;
  if (p.dtype == Dtype::BF16)
    return run_backward<bf16>(p, static_cast<const bf16*>(X), static_cast<const bf16*>(W), labels,
                              o, lse, nullptr, grad_tok, dX, dW, ws, st, timer);
  return run_backward<float>(p, static_cast<const float*>(X), static_cast<const float*>(W), labels,
                             o, lse, stat, grad_tok, dX, dW, ws, st, timer);
}

hipError_t launch_scale_grads(float* dX, int64_t n_dx, float* dW, int64_t n_dw, const float* g,
                              hipStream_t st, KernelTimer* timer) {
  timer->begin("scale_grads", 0.0, st);
  if (n_dx > 0) {
    k_scale<<<static_cast<unsigned>(std::min<int64_t>(4096, std::max<int64_t>(1, cdiv_i(n_dx, 1024)))),
              256, 0, st>>>(dX, n_dx, g);
    FCE_CHECK_LAUNCH();
  }
  if (n_dw > 0) {
    k_scale<<<static_cast<unsigned>(std::min<int64_t>(4096, std::max<int64_t>(1, cdiv_i(n_dw, 1024)))),
              256, 0, st>>>(dW, n_dw, g);
    FCE_CHECK_LAUNCH();
  }
  timer->end(st);
  return hipSuccess;
}

hipError_t launch_ce_logits(const CeLogitsCall& c, hipStream_t st, KernelTimer* timer) {
  Ctrl* ctrl = reinterpret_cast<Ctrl*>(c.ws + ce_off_ctrl());
  int32_t* flags = reinterpret_cast<int32_t*>(c.ws + ce_off_flags());
  float* rowloss = reinterpret_cast<float*>(c.ws + ce_off_rowloss());
  const int N = static_cast<int>(c.N), V = static_cast<int>(c.V);
  const bool none = c.o.reduction == Reduction::None;
  timer->begin("label_scan", 0.0, st);
  k_label_scan<<<1, 1024, 0, st>>>(c.labels, N, V, c.o.ignore, static_cast<int>(c.o.reduction),
                                   none ? nullptr : c.grad, ctrl, flags, std::max(N, 1), 1);
  FCE_CHECK_LAUNCH();
  timer->end(st);
  if (N > 0) {
    CeArgs a{c.Z, c.ldz, c.dZ, c.lddz, c.labels, N, V, c.o.ignore,
             static_cast<int>(c.o.reduction), c.o.eps, c.o.zloss, none ? c.grad : nullptr,
             ctrl, c.lse, none ? c.loss : rowloss, nullptr};
    timer->begin("ce_logits", 0.0, st);
    if (c.bf16 && c.dZ && (V + 7) / 8 <= kCeResidentVecs)
      k_ce_logits<bf16, false, kCeLdsIters * kCeThreads, kCeRegIters><<<N, kCeThreads, 0, st>>>(a);
    else if (c.bf16 && c.dZ)
      k_ce_logits<bf16, false, kCeCache><<<N, kCeThreads, 0, st>>>(a);
    else if (c.bf16)
      k_ce_logits<bf16, false, 0><<<N, kCeThreads, 0, st>>>(a);
    else if (c.dZ)
      k_ce_logits<float, false, kCeCache><<<N, kCeThreads, 0, st>>>(a);
    else
      k_ce_logits<float, false, 0><<<N, kCeThreads, 0, st>>>(a);
    FCE_CHECK_LAUNCH();
    timer->end(st);
  }
  if (none) return hipSuccess;
  timer->begin("loss_final", 0.0, st);
  k_loss_final<<<1, 256, 0, st>>>(rowloss, N, ctrl, c.loss);
  FCE_CHECK_LAUNCH();
  timer->end(st);
  return hipSuccess;
}

}  // namespace fce
