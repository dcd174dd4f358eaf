// gfx950 building blocks for the fused linear cross-entropy kernels:
// element traits over the MFMA instructions, global->LDS operand loaders,
// the LDS double-buffered MFMA main loop, and the XCD-aware tile order.
//
// Conventions
//   An operand is a 2-D array seen as (mn, k): mn runs along the output tile
//   (M for the MFMA "A" operand, N for "B"), k along the contraction.
//   K-major:  element (mn, k) at p[mn * ld + k]   (k contiguous)
//   MN-major: element (mn, k) at p[k * ld + mn]   (mn contiguous)
//   Both are staged into LDS as [mn][k] rows of BK elements (128 bytes: eight
//   16-byte chunks), so the MFMA fragment reads are identical for every
//   layout.  Chunk c of row r sits at chunk c ^ swz(r), swz(r) = (r ^ r>>3) & 7,
//   which keeps every 8-lane group of the three access patterns on distinct
//   banks: fragment reads (8 consecutive rows, one chunk), K-major stores (one
//   row, 8 chunks) and transposed MN-major stores (rows 8 apart, one chunk).
//   MN-major tiles are transposed in registers, VEC x VEC at a time, between
//   the 16-byte global loads and the 16-byte LDS stores.
//
//   Accumulator layouts (wave64).  fp32, 32x32 blocks: element i of lane l
//   holds row 8*(i/4) + 4*(l/32) + (i%4), column l%32.  bf16, 16x16 blocks
//   (v_mfma_f32_16x16x32_bf16): element i of lane l holds row 4*(l/16) + i,
//   column l%16.  Either way a lane owns groups of 4 consecutive rows of one
//   column; AccMap below names them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fce_tiles.h"

namespace fce {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// Hardware transcendental units (v_exp_f32 / v_log_f32, base 2).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// ------------------------------------------------------------ element traits
template <typename T>
struct Traits;

// bf16: 16x16 output blocks of v_mfma_f32_16x16x32_bf16, one per 32-deep K
// tile.  Lane l supplies row (or column) l%16 and the 8 consecutive k at
// 8*(l/16), for A and B alike, so the hardware's own k order inside the
// instruction is irrelevant.  (At equal FLOPs this instruction holds a
// higher clock under the power limit than the 32x32x16 one.)  The MFMA
// main loop for bf16 is the DMA pipeline further down.
template <>
struct Traits<bf16> {
  static constexpr int VEC = 8;  // elements per 16-byte vector
  static constexpr int MB = 16, NB = 16;
  typedef floatx4 AccT;
};

// fp32: eight v_mfma_f32_32x32x2_f32 per 16-deep K step.  Instruction j
// takes k = 8*(l/32) + j from lane l, so the same 8 consecutive elements per
// lane as the bf16 path are read from LDS.
template <>
struct Traits<float> {
  static constexpr int VEC = 4;
  static constexpr int MB = 32, NB = 32;
  typedef floatx16 AccT;
  struct Frag {
    floatx4 lo, hi;
  };
  // the 8 floats span two chunks: x and x ^ 1 (the first chunk is even)
  __device__ __forceinline__ static Frag frag(const char* row, int x) {
    Frag f;
    f.lo = *reinterpret_cast<const floatx4*>(row + (x << 4));
    f.hi = *reinterpret_cast<const floatx4*>(row + ((x ^ 1) << 4));
    return f;
  }
  __device__ __forceinline__ static void mma(floatx16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[0], b.lo[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[1], b.lo[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[2], b.lo[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[3], b.lo[3], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[0], b.hi[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[1], b.hi[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[2], b.hi[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[3], b.hi[3], c, 0, 0, 0);
  }
};

// ------------------------------------------------------------------ config
template <class S, typename T>
struct Cfg {
  typedef T Elem;
  typedef Traits<T> Tr;
  static constexpr int BM = S::BM, BN = S::BN, BK = S::BK;
  static constexpr int WAVES_M = S::WAVES_M, WAVES_N = S::WAVES_N, NT = S::NT;
  static constexpr int VEC = Tr::VEC;
  static constexpr int LDK = BK;  // LDS row pitch (elements): 128 bytes, swizzled
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int MB = Tr::MB, NB = Tr::NB;  // MFMA output block
  static constexpr int FM = WTM / MB, FN = WTN / NB;
  static constexpr int NV = MB * NB / 64;         // accumulator values per lane per block
  static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_ELEMS = 2 * STAGE;
  static_assert(BK % 16 == 0 && WTM % MB == 0 && WTN % NB == 0, "tile shape");
  static_assert(BK * sizeof(T) == 128, "LDS rows are eight 16-byte chunks");
  static_assert(LDS_ELEMS * sizeof(T) <= 160 * 1024, "gfx950 LDS is 160 KiB per workgroup");
};

template <typename T>
struct Opnd {
  const T* p;
  int64_t ld;  // leading dimension in elements
  int mn_ext;  // vectors starting at or beyond this mn are read as zero
  int k_ext;   // k at or beyond this are read as zero (K-major: multiple of VEC)
};

// Chunk swizzle of LDS row r.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ void transpose_block(const u32x4 (&in)[8], u32x4 (&out)[8]) {
  // 8x8 of 16-bit: in[r] holds row r (k), element c in word c/2, half c%2.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = in[2 * q][j >> 1];
      const uint32_t hi = in[2 * q + 1][j >> 1];
      out[j][q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
  }
}

__device__ __forceinline__ void transpose_block(const u32x4 (&in)[4], u32x4 (&out)[4]) {
  // 4x4 of 32-bit.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) out[j][q] = in[q][j];
  }
}

// Buffer resource covering `bytes` from `base` (gfx9 raw buffer: stride 0,
// word 3 = 0x00020000).  Loads at offsets >= the record count return zero,
// which supplies the zero fill of ragged tiles without branches.  The count
// is clamped to 2^31 - 1 so that kOOB below is always out of range.
constexpr uint32_t kOOB = 0x80000000u;

// s_waitcnt immediate that waits for vmcnt <= n (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14) and leaves expcnt / lgkmcnt unconstrained.
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// `base` and `bytes` must be uniform over the wave (they are moved to
// scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // clamp to [0, 2^31 - 1] with 32-bit compares (scalar ALU has no signed
  // 64-bit less-than)
  // (the empty asm keeps the halves apart in scalar registers, so the
  // compares stay 32-bit scalar ones: there is no scalar 64-bit less-than)
  const uint64_t u = static_cast<uint64_t>(bytes);
  uint32_t uhi = static_cast<uint32_t>(u >> 32), ulo = static_cast<uint32_t>(u);
  asm("" : "+s"(uhi), "+s"(ulo));
  const uint32_t n = (uhi & 0x80000000u) ? 0u : ((uhi != 0u || ulo > 0x7fffffffu) ? 0x7fffffffu : ulo);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  void* bs = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(bs, 0, static_cast<int>(n), 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Global -> register -> LDS staging of one ROWS x BK operand tile.  Each K
// step gets a buffer descriptor based at the step's first element, so all
// per-lane offsets are small constants of the tile.
template <class C, int ROWS, bool KMAJOR>
struct Loader;

template <class C, int ROWS>
struct Loader<C, ROWS, true> {
  typedef typename C::Elem T;
  static constexpr int VEC = C::VEC;
  static constexpr int VPR = C::BK / VEC;      // vectors per row
  static constexpr int RSTEP = C::NT / VPR;    // rows between a thread's vectors
  static constexpr int NREG = ROWS / RSTEP;
  static_assert(C::NT % VPR == 0 && ROWS % RSTEP == 0, "K-major loader geometry");
  typedef u32x4 Regs[NREG];
  const T* tile;     // element (mn0, 0)
  int64_t rows_left; // valid rows from mn0
  uint32_t off0, rstep_bytes;
  int row0, kv;

  __device__ __forceinline__ void init(const Opnd<T>& op, int mn0, int tid) {
    kv = (tid % VPR) * VEC;
    row0 = tid / VPR;
    tile = op.p + static_cast<int64_t>(mn0) * op.ld;
    rows_left = op.mn_ext - mn0;
    off0 = static_cast<uint32_t>((row0 * op.ld + kv) * static_cast<int64_t>(sizeof(T)));
    rstep_bytes = static_cast<uint32_t>(RSTEP * op.ld * static_cast<int64_t>(sizeof(T)));
  }
  // `live` false turns every load into an out-of-range (zero, no traffic) access
  __device__ __forceinline__ void load(Regs& r, const Opnd<T>& op, int k0, bool live = true) const {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(tile + k0, (rows_left * op.ld - k0) * static_cast<int64_t>(sizeof(T)));
    // a ragged last K step parks the lanes past k_ext beyond the record count
    // (kOOB + i * rstep stays below 2^32 and above every valid count)
    const uint32_t off = (live && k0 + kv < op.k_ext) ? off0 : kOOB;
#pragma unroll
    for (int i = 0; i < NREG; ++i) r[i] = buf_load16(rs, off + i * rstep_bytes);
  }
  __device__ __forceinline__ void store(const Regs& r, T* lds) const {
    char* base = reinterpret_cast<char*>(lds);
    const int c = kv / VEC;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      const int row = row0 + i * RSTEP;
      *reinterpret_cast<u32x4*>(base + row * 128 + ((c ^ swz(row)) << 4)) = r[i];
    }
  }
};

template <class C, int ROWS>
struct Loader<C, ROWS, false> {
  typedef typename C::Elem T;
  static constexpr int VEC = C::VEC;
  static constexpr int BPR = ROWS / VEC;           // VEC x VEC blocks along mn
  static constexpr int KSTEP = C::NT / BPR;        // k-blocks between a thread's blocks
  static constexpr int NBLK = (C::BK / VEC) / KSTEP;
  static constexpr int NREG = NBLK * VEC;
  static_assert(C::NT % BPR == 0 && (C::BK / VEC) % KSTEP == 0 && NBLK >= 1,
                "MN-major loader geometry");
  typedef u32x4 Regs[NREG];
  const T* tile;  // element (mn0, k = 0)
  int mn0;
  uint32_t off0, ld_bytes;
  int mb, kb0;

  __device__ __forceinline__ void init(const Opnd<T>& op, int mn0_, int tid) {
    mn0 = mn0_;
    mb = (tid % BPR) * VEC;
    kb0 = (tid / BPR) * VEC;
    tile = op.p + mn0;
    ld_bytes = static_cast<uint32_t>(op.ld * static_cast<int64_t>(sizeof(T)));
    off0 = static_cast<uint32_t>((kb0 * op.ld + mb) * static_cast<int64_t>(sizeof(T)));
  }
  __device__ __forceinline__ void load(Regs& r, const Opnd<T>& op, int k0, bool live = true) const {
    // rows k >= k_ext lie past the record count and read as zero; columns
    // past mn_ext only feed output columns that are never stored
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(tile + static_cast<int64_t>(k0) * op.ld,
                  live ? ((op.k_ext - k0) * op.ld - mn0) * static_cast<int64_t>(sizeof(T)) : 0);
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
#pragma unroll
      for (int rr = 0; rr < VEC; ++rr)
        r[b * VEC + rr] = buf_load16(rs, off0 + (b * KSTEP * VEC + rr) * ld_bytes);
  }
  __device__ __forceinline__ void store(const Regs& r, T* lds) const {
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      u32x4 in[VEC], out[VEC];
#pragma unroll
      for (int rr = 0; rr < VEC; ++rr) in[rr] = r[b * VEC + rr];
      transpose_block(in, out);
      const int c = (kb0 + b * KSTEP * VEC) / VEC;
      char* base = reinterpret_cast<char*>(lds);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const int row = mb + j;
        *reinterpret_cast<u32x4*>(base + row * 128 + ((c ^ swz(row)) << 4)) = out[j];
      }
    }
  }
};

template <class C>
struct Acc {
  typename C::Tr::AccT v[C::FM][C::FN];
};

// Which output elements a lane holds: in block (fm, fn) of the wave tile,
// value 4 g + q (g < NGRP, q < 4) is row fm * MB + row(lane, g) + q,
// column fn * NB + col(lane).
template <class C>
struct AccMap {
  static constexpr int MB = C::MB, NB = C::NB;
  static constexpr int NGRP = C::NV / 4;  // groups of 4 consecutive rows
  __device__ __forceinline__ static int row(int lane, int g) {
    return 4 * (64 / NB) * g + 4 * (lane / NB);
  }
  __device__ __forceinline__ static int col(int lane) { return lane % NB; }
};

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x0002, kSchedMFMA = 0x0008, kSchedVMEMRead = 0x0020,
              kSchedDSRead = 0x0100, kSchedDSWrite = 0x0200;

// One BM x BN output tile: acc = A[m0:m0+BM, 0:K] . B[n0:n0+BN, 0:K]^T.
//
// Pipeline per BK-deep tile (two LDS stages, two register sets of MFMA
// fragments): the global loads of tile t+1 are issued during the first
// 16-deep sub-step of tile t; every sub-step reads the next sub-step's
// fragments from LDS while its own MFMAs run; the last sub-step writes tile
// t+1 into the other LDS stage between its MFMAs; one barrier per tile.  The
// interleaving is pinned with scheduling-group barriers so the MFMA pipe is
// not left waiting on an LDS round trip it could have overlapped.  Ends with
// a barrier, so LDS may be reused after it.
template <class C, bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void gemm_tile(Acc<C>& acc, const Opnd<typename C::Elem>& A,
                                          const Opnd<typename C::Elem>& B, int m0, int n0, int K,
                                          typename C::Elem* lds0, typename C::Elem* lds1,
                                          int tid) {
  typedef typename C::Elem T;
  typedef typename C::Tr Tr;
  constexpr int KS = C::BK / 16;
  constexpr int NMMA = C::FM * C::FN;  // MFMA instructions per sub-step (bf16)
  constexpr int NFRAG = C::FM + C::FN;
  typedef Loader<C, C::BM, A_KMAJOR> LA;
  typedef Loader<C, C::BN, B_KMAJOR> LB;
  constexpr int NVMEM = LA::NREG + LB::NREG;
  static_assert(KS % 2 == 0, "fragment sets alternate within a tile");
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int i = 0; i < C::NV; ++i) acc.v[fm][fn][i] = 0.0f;
  const int nk = (K + C::BK - 1) / C::BK;
  if (nk <= 0) return;

  LA la;
  LB lb;
  la.init(A, m0, tid);
  lb.init(B, n0, tid);
  typename LA::Regs ra;
  typename LB::Regs rb;
  la.load(ra, A, 0);
  lb.load(rb, B, 0);
  la.store(ra, lds0);
  lb.store(rb, lds0 + C::A_ELEMS);
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // Fragment f of sub-step k16 covers k = 16*k16 + 8*(lane/32) .. +8 of row
  // base + 32*f + lane%32: its first chunk is k16*CPS + (lane/32)*CPH.
  constexpr int CPH = 8 * static_cast<int>(sizeof(T)) / 16;  // chunks per half fragment
  constexpr int CPS = 2 * CPH;                                // chunks per sub-step
  const int hl = lane >> 5;
  const int a_row = wm * C::WTM + (lane & 31);
  const int b_row = wn * C::WTN + (lane & 31);
  int ax[C::FM], bx[C::FN];  // (first chunk of sub-step 0) ^ swizzle, per fragment row
#pragma unroll
  for (int f = 0; f < C::FM; ++f) ax[f] = (hl * CPH) ^ swz(a_row + 32 * f);
#pragma unroll
  for (int f = 0; f < C::FN; ++f) bx[f] = (hl * CPH) ^ swz(b_row + 32 * f);

  typename Tr::Frag fa[2][C::FM], fb[2][C::FN];
  auto read_frags = [&](int set, const T* As, int k16) {
    const char* Ab = reinterpret_cast<const char*>(As);
    const char* Bb = reinterpret_cast<const char*>(As + C::A_ELEMS);
#pragma unroll
    for (int f = 0; f < (C::FM > C::FN ? C::FM : C::FN); ++f) {
      // k16 * CPS only touches chunk bits above the lane's own, so XOR composes
      if (f < C::FM) fa[set][f] = Tr::frag(Ab + (a_row + 32 * f) * 128, ax[f] ^ (k16 * CPS));
      if (f < C::FN) fb[set][f] = Tr::frag(Bb + (b_row + 32 * f) * 128, bx[f] ^ (k16 * CPS));
    }
  };
  auto mma_set = [&](int set) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) Tr::mma(acc.v[fm][fn], fa[set][fm], fb[set][fn]);
  };
  const bool pin = sizeof(T) == 2;  // pin the bf16 interleaving; fp32 is left to the compiler

  read_frags(0, lds0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const T* As = (kt & 1) ? lds1 : lds0;
    T* nxt = (kt & 1) ? lds0 : lds1;
    // prefetch tile kt+1; past the last tile the loads are out of range (no
    // traffic) and the stores fill an LDS stage nobody reads
    const bool live = kt + 1 < nk;
    la.load(ra, A, (kt + 1) * C::BK, live);
    lb.load(rb, B, (kt + 1) * C::BK, live);
#pragma unroll
    for (int k16 = 0; k16 < KS; ++k16) {
      const int cur = k16 & 1;
      if (k16 + 1 < KS) read_frags(cur ^ 1, As, k16 + 1);
      mma_set(cur);
      if (k16 + 1 == KS) {
        la.store(ra, nxt);
        lb.store(rb, nxt + C::A_ELEMS);
      }
      if (pin) {
        if (k16 == 0) {
#pragma unroll
          for (int g = 0; g < NFRAG; ++g) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVMEMRead, NVMEM / NFRAG, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, NMMA - NFRAG, 0);
        } else if (k16 + 1 < KS) {
#pragma unroll
          for (int g = 0; g < NFRAG; ++g) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, NMMA - NFRAG, 0);
        } else {
#pragma unroll
          for (int g = 0; g < NMMA / 2; ++g) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVALU, 8, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSWrite, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, NMMA / 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    read_frags(0, nxt, 0);
  }
}

// ===================================================== bf16 DMA main loop
// gfx950 path for bf16: operand tiles go straight from global memory into LDS
// with buffer_load_dwordx4 ... lds (lane l of a wave lands at M0 + 16 l), so
// no registers stage them and nothing is transposed in registers.
//
// LDS layouts (per stage, BK = 32):
//   K-major operand:  [ROWS][32] bf16, 64-byte rows of four 16-byte chunks;
//                     chunk c of row r at chunk c ^ km_swz(r).
//   MN-major operand: [32][ROWS] bf16, untransposed rows of k; 16-byte chunk c
//                     of row k at chunk c ^ mn_swz(k).
// Fragment reads (16x16x32 MFMA: lane l takes row l%16, k = 8 (l/16) .. +7):
// K-major with one ds_read_b128; MN-major with two ds_read_b64_tr_b16.  In
// each 16-lane group that instruction hands lane j element j%4 of the 8-byte
// chunks addressed by lanes j/4 + 4q (q = 0..3), so lane a addressing k-row
// 8 (l/16) + a/4 (then + 4) at column 4 (a%4) of the fragment gives lane j
// the 8 consecutive k of column j, the same fragment a K-major read gives.
// Both swizzles are free of LDS bank conflicts for these reads (measured with
// SQ_LDS_BANK_CONFLICT); for the b64 transpose reads the reasoning is 64
// banks of 4 bytes and 32-lane phases: k-rows 8G + q for two G and four q,
// 32 contiguous bytes each, land on distinct banks.
// Pipeline: STAGES LDS stages; the loads of tile t+STAGES-1 are issued at the
// start of tile t, so each tile's data has STAGES-2 tiles of MFMA work to
// land before the barrier that publishes it.

template <int ROWS, bool KMAJOR, int NT_>
struct DmaOperand;

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Swizzle (in 16-byte chunks) of row `row` of a K-major LDS tile.  Chosen by
// measurement (SQ_LDS_BANK_CONFLICT of ds_read_b128 with the 16x16 fragment
// pattern below: zero for this one, about four conflict cycles per read for
// the row bits (r >> 2) & 3, r & 3 or none).
__host__ __device__ constexpr int km_swz(int row) { return (row >> 1) & 3; }

// Swizzle (in 16-byte chunks) of k-row `krow` of an MN-major LDS tile.
__host__ __device__ constexpr int mn_swz(int krow) {
  return (4 * (krow & 3)) ^ (2 * ((krow >> 3) & 1));
}

template <int ROWS, int NT_>
struct DmaOperand<ROWS, true, NT_> {
  static constexpr int BK = 32, NT = NT_;
  static constexpr int BYTES = ROWS * BK * 2;       // per stage
  static constexpr int NI = BYTES / (NT * 16);      // DMA instructions per thread per tile
  static constexpr int ROWS_PER_I = NT * 16 / 64;   // rows per instruction round
  static_assert(NI >= 1 && BYTES % (NT * 16) == 0, "K-major DMA geometry");
  const bf16* tile;
  int64_t rows_left;
  uint32_t voff0, istep;
  int kc;  // k offset of this thread's chunk

  __device__ __forceinline__ void init(const Opnd<bf16>& op, int mn0, int tid) {
    const int row = tid >> 2;              // (16 tid) / 64
    const int c = (tid & 3) ^ km_swz(row);
    kc = c * 8;
    tile = op.p + static_cast<int64_t>(mn0) * op.ld;
    rows_left = op.mn_ext - mn0;
    voff0 = static_cast<uint32_t>((row * op.ld + kc) * 2);
    istep = static_cast<uint32_t>(ROWS_PER_I * op.ld * 2);
  }
  // kfull (a constant at every call): K is a whole number of 32-deep tiles,
  // so no lane's chunk ever starts past k_ext and a dead load (live false)
  // needs no per-lane offset: an empty descriptor returns its zeros.
  __device__ __forceinline__ void load(char* stage, int wave, const Opnd<bf16>& op, int k0,
                                       bool live, bool kfull) const {
    load_rows(stage, wave, op, tile, rows_left, k0, live, kfull);
  }
  // The same load for the tile whose first row is mn0 (any tile of `op`).
  __device__ __forceinline__ void load_at(char* stage, int wave, const Opnd<bf16>& op, int mn0,
                                          int k0, bool live, bool kfull) const {
    load_rows(stage, wave, op, op.p + static_cast<int64_t>(mn0) * op.ld, op.mn_ext - mn0, k0,
              live, kfull);
  }
  __device__ __forceinline__ void load_rows(char* stage, int wave, const Opnd<bf16>& op,
                                            const bf16* tile_, int64_t rows_left_, int k0,
                                            bool live, bool kfull) const {
    const int64_t count = (rows_left_ * op.ld - k0) * 2;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile_ + k0, (kfull && !live) ? 0 : count);
    const uint32_t off = kfull ? voff0 : ((live && k0 + kc < op.k_ext) ? voff0 : kOOB);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_ptr_t)(stage + i * NT * 16 + wave * 1024), 16, off + i * istep, 0, 0, 0);
  }
};

template <int ROWS, int NT_>
struct DmaOperand<ROWS, false, NT_> {
  static constexpr int BK = 32, NT = NT_;
  static constexpr int ROWB = ROWS * 2;              // bytes per k-row
  static constexpr int BYTES = BK * ROWB;
  static constexpr int NI = BYTES / (NT * 16);
  static constexpr int KROWS_PER_I = NT * 16 / ROWB;
  // mn_swz has period 16 in the k-row: instructions 16 k-rows apart share the
  // vector offset; with 8 k-rows per round, odd rounds need a second one
  static constexpr int NV = (KROWS_PER_I % 16 == 0 || NI == 1) ? 1 : 2;
  static_assert(ROWB % 1024 == 0 || 1024 % ROWB == 0, "k-rows tile the 1 KiB DMA blocks");
  static_assert(NI >= 1 && BYTES % (NT * 16) == 0, "MN-major DMA geometry");
  static_assert(ROWB >= 256 && KROWS_PER_I % 8 == 0, "swizzle geometry");
  const bf16* tile;
  int mn0;
  uint32_t voff[NV], istep;  // round v's offset; bytes per NV rounds of k-rows

  __device__ __forceinline__ void init(const Opnd<bf16>& op, int mn0_, int tid) {
    mn0 = mn0_;
    tile = op.p + mn0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int byte = (v * NT + tid) * 16;  // position in the stage of round v
      const int krow = byte / ROWB;
      const int c = ((byte % ROWB) / 16) ^ mn_swz(krow);
      voff[v] = static_cast<uint32_t>((krow * op.ld + c * 8) * 2);
    }
    istep = static_cast<uint32_t>(NV * KROWS_PER_I * op.ld * 2);
  }
  __device__ __forceinline__ void load(char* stage, int wave, const Opnd<bf16>& op, int k0,
                                       bool live, bool /*kfull*/) const {
    // rows k >= k_ext lie past the record count and read as zero
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(tile + static_cast<int64_t>(k0) * op.ld,
                  live ? ((op.k_ext - k0) * op.ld - mn0) * static_cast<int64_t>(2) : 0);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_ptr_t)(stage + i * NT * 16 + wave * 1024), 16,
          voff[i % NV] + (i / NV) * istep, 0, 0, 0);
  }
};

// Per-lane fragment addressing of one operand (relative to the stage base):
// fragment f covers rows wave_base + 16 f .. +15 and the whole K tile.
template <int ROWS, bool KMAJOR, int NF>
struct FragAddr;

template <int ROWS, int NF>
struct FragAddr<ROWS, true, NF> {
  int off;  // byte offset of fragment 0
  __device__ __forceinline__ void init(int wave_base, int lane) {
    const int r = wave_base + (lane & 15);
    const int x = (lane >> 4) ^ km_swz(r);
    off = r * 64 + 16 * x;
  }
  __device__ __forceinline__ bf16x8 read(const char* stage, int f) const {
    // 16 f rows further down keep the same km_swz
    return *reinterpret_cast<const bf16x8*>(stage + off + f * 16 * 64);
  }
};

template <int ROWS, int NF>
struct FragAddr<ROWS, false, NF> {
  static constexpr int ROWB = ROWS * 2;
  static_assert((NF & (NF - 1)) == 0 && NF <= 8, "power-of-two fragment count");
  int off0;  // byte offset of the first transpose read of fragment 0
  __device__ __forceinline__ void init(int wave_base, int lane) {
    const int a = lane & 15;
    const int krow = 8 * (lane >> 4) + (a >> 2);  // the second read is 4 k-rows on,
    const int sw = mn_swz(krow);                  // with the same swizzle
    const int mn = wave_base + 4 * (a & 3);
    off0 = krow * ROWB + 16 * ((mn >> 3) ^ sw) + (mn & 7) * 2;
  }
  // Fragment f sits 16 f columns on: with wave_base a multiple of 16 NF the
  // chunk index gains 2 f without carries, and the swizzle (bits 1..3 of the
  // chunk index) commutes with that, so its offset is off0 ^ 32 f.
  __device__ __forceinline__ bf16x8 read(const char* stage, int f) const {
    // one v_xor per read (volatile: not hoisted into a register per fragment)
    int o = off0;
    if (f != 0) asm volatile("v_xor_b32 %0, %1, %2" : "=v"(o) : "i"(32 * f), "v"(off0));
    const char* p = stage + o;
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(p));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) shortx4*)(p + 4 * ROWB));
    const shortx4 v[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// The four LDS stages of the DMA pipeline.  They are distinct objects so the
// compiler can tell a DMA into one stage from a read of another (it tracks
// LDS-DMA completion per object); kernels declare them with
// FCE_DMA_STAGES(name) and hand them over as a DmaStages.
struct DmaStages {
  char* s[4];
};
#define FCE_DMA_STAGES(name)                                                      \
  __shared__ __attribute__((aligned(16))) char name##0[32768], name##1[32768],    \
      name##2[32768], name##3[32768];                                             \
  const ::fce::DmaStages name = {{name##0, name##1, name##2, name##3}}

// Waits for this wave's LDS reads and all but the newest `n` vector-memory
// operations, then joins the workgroup barrier.  (__syncthreads would also
// drain every in-flight prefetch.)
template <int N>
__device__ __forceinline__ void barrier_after_vmcnt() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N) & ~(0xF << 8));  // and lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// The per-wave machinery of the DMA pipeline for one BM x BN tile shape:
// operand DMA, fragment reads, MFMAs and their order within one 32-deep K
// tile.  Any wave layout C::WAVES_M x C::WAVES_N whose wave tile is a
// multiple of 16 x 16; 256 or 512 threads.
//
// Fragment registers: the operand with more fragments per wave ("rolling",
// NRL of them) has ONE register set; the other ("double", NDB) has two.  The
// MFMAs of a K tile run as NRL rows of NDB (row r uses rolling fragment r),
// and rolling fragment r of the next K tile is read into its register as
// soon as row r has issued, so the reads of the next tile overlap the
// current tile's MFMAs without a second rolling set.  Scheduling barriers
// between rows keep every read after the last use of the register it
// overwrites.  Odd rows walk their double fragments in reverse, so that
// every MFMA of a K tile shares one operand register with the one before
// it, also across rows: on random data the matrix pipes run power-limited,
// and fewer operand changes per MFMA let the clock rise (the step at
// 8192 x 4096 x 128256 took 25.73 instead of 25.99 ms, every product
// faster).  Each accumulator still receives its MFMAs in K order, so the
// results are bitwise the same.
template <class C, bool A_KMAJOR, bool B_KMAJOR, bool KFULL>
struct DmaEngine {
  static constexpr int S = 4, BK = 32;
  static constexpr int B_OFF = C::BM * BK * 2;
  static constexpr int FM = C::FM, FN = C::FN;
  typedef DmaOperand<C::BM, A_KMAJOR, C::NT> DA;
  typedef DmaOperand<C::BN, B_KMAJOR, C::NT> DB;
  static constexpr int NL = DA::NI + DB::NI;  // DMA instructions per thread per K tile
  static constexpr bool ROLL_A = FM >= FN;
  static constexpr int NRL = ROLL_A ? FM : FN;  // rolling fragments = MFMA rows
  static constexpr int NDB = ROLL_A ? FN : FM;  // double-buffered fragments = MFMAs per row
  static_assert(C::MB == 16 && C::NB == 16 && NRL >= 2, "16x16 blocks, two rows at least");
  static_assert(C::BM * BK * 2 + C::BN * BK * 2 <= 32768, "one K tile per 32 KiB stage");

  DA da;
  DB db;
  FragAddr<C::BM, A_KMAJOR, FM> fa_addr;
  FragAddr<C::BN, B_KMAJOR, FN> fb_addr;
  bf16x8 fr[NRL], fd[2][NDB];
  int wave;

  __device__ __forceinline__ void init(const Opnd<bf16>& A, const Opnd<bf16>& B, int m0, int n0,
                                       int tid) {
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    da.init(A, m0, tid);
    db.init(B, n0, tid);
    fa_addr.init(wm * C::WTM, lane);
    fb_addr.init(wn * C::WTN, lane);
  }
  __device__ __forceinline__ bf16x8 read_a(const char* stage, int f) const {
    return fa_addr.read(stage, f);
  }
  __device__ __forceinline__ bf16x8 read_b(const char* stage, int f) const {
    return fb_addr.read(stage + B_OFF, f);
  }
  __device__ __forceinline__ void read_roll(const char* stage, int r) {
    fr[r] = ROLL_A ? read_a(stage, r) : read_b(stage, r);
  }
  __device__ __forceinline__ void read_dbl(int set, const char* stage, int d) {
    fd[set][d] = ROLL_A ? read_b(stage, d) : read_a(stage, d);
  }
  // Every fragment of the K tile in `stage` (double ones into set `set`).
  __device__ __forceinline__ void read_all(int set, const char* stage) {
#pragma unroll
    for (int r = 0; r < NRL; ++r) read_roll(stage, r);
#pragma unroll
    for (int d = 0; d < NDB; ++d) read_dbl(set, stage, d);
  }
  __device__ __forceinline__ void mma_row(Acc<C>& acc, int set, int r) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      const int d = (r & 1) ? NDB - 1 - i : i;  // odd rows in reverse
      const int fm = ROLL_A ? r : d, fn = ROLL_A ? d : r;
      const bf16x8& a = ROLL_A ? fr[r] : fd[set][d];
      const bf16x8& b = ROLL_A ? fd[set][d] : fr[r];
      acc.v[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc.v[fm][fn], 0, 0, 0);
    }
  }
  // The barrier that publishes the next K tile comes after the first HALF
  // rows, so the LDS reads it waits for (lgkmcnt(0)) have half a tile of
  // MFMAs to land.
  static constexpr int HALF = NRL / 2;
  // Row of the MFMA order before which double fragment d of the next tile is
  // read (rows HALF .. NRL-1, spread evenly).
  __device__ __forceinline__ static constexpr int dbl_row(int d) {
    return HALF + (d * (NRL - HALF)) / NDB;
  }
  // One K tile whose fragments are already in registers (double set SET):
  // prefetch (issue_next) into the stage of the previous tile (free since the
  // previous barrier), rows 0 .. HALF-1, publish the next tile (wait for this
  // thread's DMA of it, barrier), read its rolling fragments 0 .. HALF-1
  // (their rows are done), then rows HALF .. NRL-1, each preceded by the
  // read of the rolling fragment the previous row freed.
  template <int SET, class Issue>
  __device__ __forceinline__ void step(Acc<C>& acc, const char* nxt, Issue&& issue_next) {
    issue_next();
#pragma unroll
    for (int r = 0; r < HALF; ++r) mma_row(acc, SET, r);
    __builtin_amdgcn_sched_barrier(0);
    barrier_after_vmcnt<NL * (S - 2)>();
#pragma unroll
    for (int r = 0; r < HALF; ++r) read_roll(nxt, r);
#pragma unroll
    for (int r = HALF; r < NRL; ++r) {
      if (r > HALF) read_roll(nxt, r - 1);
#pragma unroll
      for (int d = 0; d < NDB; ++d)
        if (dbl_row(d) == r) read_dbl(SET ^ 1, nxt, d);
      mma_row(acc, SET, r);
      __builtin_amdgcn_sched_barrier(0);
    }
    read_roll(nxt, NRL - 1);
  }
};

template <class C>
__device__ __forceinline__ void zero_acc(Acc<C>& acc) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int i = 0; i < C::NV; ++i) acc.v[fm][fn][i] = 0.0f;
}

// One BM x BN bf16 output tile, operands in any layout, through the 4-stage
// DMA pipeline.  The K loop is unrolled by the stage count so every stage
// reference and fragment set is static.  When the tile count is not a
// multiple of four the last trip runs on tiles past the end, whose stages
// hold the zeros of out-of-range loads: their MFMAs add exact zeros.  Ends
// with all DMA drained and a barrier, so the stages may be reused after it.
//
// MAPPED: the K loop runs over a list of kMapBlock-long K blocks instead of
// 0 .. K-1: K counts the elements run (a multiple of kMapBlock) and K tile kt
// reads from block kmap[kt / (kMapBlock / BK)] (a device array, read with
// workgroup-uniform indices).
constexpr int kMapBlock = 256;
template <class C, bool A_KMAJOR, bool B_KMAJOR, bool KFULL, bool MAPPED = false>
__device__ __forceinline__ void gemm_tile_dma(Acc<C>& acc, const Opnd<bf16>& A,
                                              const Opnd<bf16>& B, int m0, int n0, int K,
                                              const DmaStages& st, int tid,
                                              const int* kmap = nullptr) {
  typedef DmaEngine<C, A_KMAJOR, B_KMAJOR, KFULL> E;
  constexpr int S = E::S, BK = E::BK;
  zero_acc(acc);
  const int nk = (K + BK - 1) / BK;
  if (nk <= 0) return;
  E e;
  e.init(A, B, m0, n0, tid);
  auto koff = [&](int kt) -> int {
    if constexpr (MAPPED) {
      constexpr int KB = kMapBlock / BK;
      static_assert(kMapBlock % BK == 0, "whole K tiles per mapped block");
      return kt < nk ? kmap[kt / KB] * kMapBlock + (kt % KB) * BK : 0;
    } else {
      return kt * BK;
    }
  };
  auto issue = [&](char* stage, int kt) {
    const bool live = kt < nk;
    const int k0 = koff(kt);
    e.da.load(stage, e.wave, A, k0, live, KFULL);
    e.db.load(stage + E::B_OFF, e.wave, B, k0, live, KFULL);
  };
  issue(st.s[0], 0);
  issue(st.s[1], 1);
  issue(st.s[2], 2);
  barrier_after_vmcnt<E::NL * (S - 2)>();
  e.read_all(0, st.s[0]);
  for (int kt = 0; kt < nk; kt += S) {
    e.template step<0>(acc, st.s[1], [&] { issue(st.s[3], kt + 3); });
    e.template step<1>(acc, st.s[2], [&] { issue(st.s[0], kt + 4); });
    e.template step<0>(acc, st.s[3], [&] { issue(st.s[1], kt + 5); });
    e.template step<1>(acc, st.s[0], [&] { issue(st.s[2], kt + 6); });
  }
  // the prefetches past the last tile still write (zeros) into LDS: drain them
  barrier_after_vmcnt<0>();
}

// Ping-pong K loop: the two wave groups (wm = 0 and wm = 1, one wave of each
// per SIMD) alternate between an MFMA phase (a whole K tile from registers)
// and a memory phase (the next tile's fragments into the single register
// set, the DMA share of a tile three ahead), half a tile apart, with a
// barrier per half step: while one group synchronises, the other feeds the
// matrix pipe.  Group A reads tile 0 before the loop; then at half step 2t
// A computes tile t while B loads tile t, at 2t+1 A loads tile t+1 while B
// computes tile t.
template <class C, bool A_KMAJOR, bool B_KMAJOR, bool KFULL>
__device__ __forceinline__ void gemm_tile_pp(Acc<C>& acc, const Opnd<bf16>& A,
                                             const Opnd<bf16>& B, int m0, int n0, int K,
                                             const DmaStages& st, int tid) {
  typedef DmaEngine<C, A_KMAJOR, B_KMAJOR, KFULL> E;
  constexpr int BK = E::BK, NL = E::NL;
  static_assert(C::WAVES_M == 2 && E::S == 4, "two wave groups, four stages");
  zero_acc(acc);
  const int nk = (K + BK - 1) / BK;
  if (nk <= 0) return;
  E e;
  e.init(A, B, m0, n0, tid);
  const bool ga = (e.wave / C::WAVES_N) == 0;  // group A (wave-uniform)
  // stage of tile kt is kt % 4; the loop is unrolled by 4 so every stage
  // index is a constant
  auto issue = [&](char* stage, int kt) {
    const bool live = kt < nk;
    e.da.load(stage, e.wave, A, kt * BK, live, KFULL);
    e.db.load(stage + E::B_OFF, e.wave, B, kt * BK, live, KFULL);
  };
  auto mma_all = [&]() {
#pragma unroll
    for (int r = 0; r < E::NRL; ++r) e.mma_row(acc, 0, r);
  };
  issue(st.s[0], 0);
  issue(st.s[1], 1);
  issue(st.s[2], 2);
  if (ga) {
    issue(st.s[3], 3);
    barrier_after_vmcnt<3 * NL>();
    e.read_all(0, st.s[0]);
    for (int t = 0; t < nk; t += 4) {
#define PP_A(J)                                                             \
      if (t + J >= nk) break;                                               \
      mma_all();                                                            \
      __builtin_amdgcn_sched_barrier(0);                                    \
      barrier_after_vmcnt<2 * NL>();                                        \
      if (t + J + 1 < nk) e.read_all(0, st.s[(J + 1) & 3]);                 \
      issue(st.s[J & 3], t + J + 4);                                        \
      __builtin_amdgcn_sched_barrier(0);                                    \
      barrier_after_vmcnt<3 * NL>();
      PP_A(0) PP_A(1) PP_A(2) PP_A(3)
#undef PP_A
    }
  } else {
    barrier_after_vmcnt<2 * NL>();
    for (int t = 0; t < nk; t += 4) {
#define PP_B(J)                                                             \
      if (t + J >= nk) break;                                               \
      e.read_all(0, st.s[J & 3]);                                           \
      issue(st.s[(J + 3) & 3], t + J + 3);                                  \
      __builtin_amdgcn_sched_barrier(0);                                    \
      barrier_after_vmcnt<2 * NL>();                                        \
      mma_all();                                                            \
      __builtin_amdgcn_sched_barrier(0);                                    \
      barrier_after_vmcnt<2 * NL>();
      PP_B(0) PP_B(1) PP_B(2) PP_B(3)
#undef PP_B
    }
  }
  barrier_after_vmcnt<0>();
}

// Consecutive BM-row M tiles mt_begin .. mt_end-1 (K-major A, full K each)
// against one BN-column N tile of K-major B, as ONE stream of K tiles on the
// ping-pong loop of gemm_tile_pp: the DMA for the next M tile's first K
// tiles is issued while the current one finishes, so the pipeline never
// drains between M tiles.  After each M tile epi(acc, m0) consumes the
// accumulators (registers only; LDS stays with the pipeline) and they
// restart from zero.  Each group runs its epilogue at the start of one of
// its own memory phases, before the fragment reads (so that the fragment
// registers are free), while the other group's MFMAs run: group A right
// after its last MFMA phase of the M tile, group B right after the barrier
// that closes its own.  Needs K % 128 == 0: nk is then a multiple of 4, so
// the stage of a K tile is kt % 4 in every M tile and the unrolled stage
// indices hold across M tile boundaries.  Every quad of K tiles is straight-
// line code with the epilogue only in the last one: a branch with the
// accumulators live across it makes the register allocator copy them.
// Ends with all DMA drained and a barrier.
template <class C, class Epi>
__device__ __forceinline__ void gemm_stream_pp(const Opnd<bf16>& A, const Opnd<bf16>& B,
                                               int mt_begin, int mt_end, int n0, int K,
                                               const DmaStages& st, int tid, Epi&& epi) {
  typedef DmaEngine<C, true, true, true> E;
  constexpr int BK = E::BK, NL = E::NL;
  static_assert(C::WAVES_M == 2 && E::S == 4, "two wave groups, four stages");
  const int nk = K / BK;
  Acc<C> acc;
  zero_acc(acc);
  if (mt_end <= mt_begin || nk <= 0) return;
  E e;
  e.init(A, B, mt_begin * C::BM, n0, tid);
  const bool ga = (e.wave / C::WAVES_N) == 0;  // group A (wave-uniform)
  // K tile kt of M tile mt; kt < nk + 4 (past the end it wraps into the next
  // M tile, past the last M tile the load is dead)
  auto issue = [&](char* stage, int mt, int kt) {
    int m = mt, k = kt;
    if (k >= nk) {
      k -= nk;
      ++m;
    }
    const bool live = m < mt_end;
    e.da.load_at(stage, e.wave, A, (live ? m : mt_begin) * C::BM, k * BK, live, true);
    e.db.load(stage + E::B_OFF, e.wave, B, k * BK, live, true);
  };
  auto mma_all = [&]() {
#pragma unroll
    for (int r = 0; r < E::NRL; ++r) e.mma_row(acc, 0, r);
  };
  issue(st.s[0], mt_begin, 0);
  issue(st.s[1], mt_begin, 1);
  issue(st.s[2], mt_begin, 2);
  if (ga) {
    issue(st.s[3], mt_begin, 3);
    barrier_after_vmcnt<3 * NL>();
    e.read_all(0, st.s[0]);
    for (int mt = mt_begin; mt < mt_end; ++mt) {
      // four K tiles from t; the last four of the M tile end with its epilogue
      auto quad = [&](int t, auto last_c) {
        constexpr bool LAST = decltype(last_c)::value;
#define PS_A(J)                                                             \
        mma_all();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                  \
        barrier_after_vmcnt<2 * NL>();                                      \
        if constexpr (LAST && J == 3) {                                     \
          epi(acc, mt * C::BM);                                             \
          zero_acc(acc);                                                    \
          __builtin_amdgcn_sched_barrier(0);                                \
        }                                                                   \
        e.read_all(0, st.s[(J + 1) & 3]);                                   \
        issue(st.s[J & 3], mt, t + J + 4);                                  \
        __builtin_amdgcn_sched_barrier(0);                                  \
        barrier_after_vmcnt<3 * NL>();
        PS_A(0) PS_A(1) PS_A(2) PS_A(3)
#undef PS_A
      };
      for (int t = 0; t < nk - 4; t += 4) quad(t, std::false_type{});
      quad(nk - 4, std::true_type{});
    }
  } else {
    barrier_after_vmcnt<2 * NL>();
    for (int mt = mt_begin; mt < mt_end; ++mt) {
      // four K tiles from t; the last four of the M tile end with its
      // epilogue, after the barrier that closes their last MFMA phase (so
      // at the start of the group's next memory phase)
      auto quad = [&](int t, auto last_c) {
        constexpr bool LAST = decltype(last_c)::value;
#define PS_B(J)                                                             \
        e.read_all(0, st.s[J & 3]);                                         \
        issue(st.s[(J + 3) & 3], mt, t + J + 3);                            \
        __builtin_amdgcn_sched_barrier(0);                                  \
        barrier_after_vmcnt<2 * NL>();                                      \
        mma_all();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                  \
        barrier_after_vmcnt<2 * NL>();                                      \
        if constexpr (LAST && J == 3) {                                     \
          epi(acc, mt * C::BM);                                             \
          zero_acc(acc);                                                    \
          __builtin_amdgcn_sched_barrier(0);                                \
        }
        PS_B(0) PS_B(1) PS_B(2) PS_B(3)
#undef PS_B
      };
      for (int t = 0; t < nk - 4; t += 4) quad(t, std::false_type{});
      quad(nk - 4, std::true_type{});
    }
  }
  barrier_after_vmcnt<0>();
}

// gemm_stream_pp for an epilogue that stores: epi issues at least NS
// vector-memory instructions per wave (its stores, all of them
// unconditional).  gfx950 retires vector loads and stores in issue order
// against vmcnt, so a wait for a DMA issued before an epilogue's stores may
// leave those stores outstanding: its count includes them (NS more), where
// a count of DMA issues alone would hold the wave until the newer prefetches
// and the stores had landed.  After an epilogue that is the last wait of
// group A's epilogue quad and the first four waits of the next quad of
// either group.  So that the first M tile runs the same code,
// each wave first issues NS stores that the hardware drops (a buffer
// resource of zero bytes) where an epilogue's stores would sit, and the
// prologue waits count them too.  Needs K % 128 == 0 and K >= 256 (two quads
// or more per M tile, so a quad never both follows and holds an epilogue).
template <class C, int NS, class Epi>
__device__ __forceinline__ void gemm_stream_pp_st(const Opnd<bf16>& A, const Opnd<bf16>& B,
                                                  int mt_begin, int mt_end, int n0, int K,
                                                  const DmaStages& st, int tid, Epi&& epi) {
  typedef DmaEngine<C, true, true, true> E;
  constexpr int BK = E::BK, NL = E::NL;
  static_assert(C::WAVES_M == 2 && E::S == 4, "two wave groups, four stages");
  static_assert(NS > 0 && 3 * NL + NS <= 63, "vmcnt counts up to 63");
  const int nk = K / BK;
  Acc<C> acc;
  zero_acc(acc);
  if (mt_end <= mt_begin || nk < 8) return;
  E e;
  e.init(A, B, mt_begin * C::BM, n0, tid);
  const bool ga = (e.wave / C::WAVES_N) == 0;  // group A (wave-uniform)
  auto issue = [&](char* stage, int mt, int kt) {
    int m = mt, k = kt;
    if (k >= nk) {
      k -= nk;
      ++m;
    }
    const bool live = m < mt_end;
    e.da.load_at(stage, e.wave, A, (live ? m : mt_begin) * C::BM, k * BK, live, true);
    e.db.load(stage + E::B_OFF, e.wave, B, k * BK, live, true);
  };
  auto mma_all = [&]() {
#pragma unroll
    for (int r = 0; r < E::NRL; ++r) e.mma_row(acc, 0, r);
  };
  issue(st.s[0], mt_begin, 0);
  issue(st.s[1], mt_begin, 1);
  issue(st.s[2], mt_begin, 2);
  {
    // NS dropped stores in place of a previous epilogue's (distinct offsets
    // and volatile, so that the compiler keeps every one of them)
    const __amdgpu_buffer_rsrc_t none = make_rsrc(A.p, 0);
    constexpr int kVolatile = static_cast<int>(1u << 31);  // intrinsic aux bit 31
#pragma unroll
    for (int i = 0; i < NS; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 4 * i, 0, kVolatile);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (ga) {
    issue(st.s[3], mt_begin, 3);
    barrier_after_vmcnt<3 * NL + NS>();
    e.read_all(0, st.s[0]);
    for (int mt = mt_begin; mt < mt_end; ++mt) {
      // four K tiles from t; LAST: the last four of the M tile, ending with
      // its epilogue; AFTER: the first four, after the previous epilogue
      auto quad = [&](int t, auto last_c, auto after_c) {
        constexpr bool LAST = decltype(last_c)::value;
        constexpr bool AFTER = decltype(after_c)::value;
#define PS_A(J)                                                             \
        mma_all();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                  \
        barrier_after_vmcnt<2 * NL + ((AFTER && J < 2) ? NS : 0)>();        \
        if constexpr (LAST && J == 3) {                                     \
          epi(acc, mt * C::BM);                                             \
          zero_acc(acc);                                                    \
          __builtin_amdgcn_sched_barrier(0);                                \
        }                                                                   \
        e.read_all(0, st.s[(J + 1) & 3]);                                   \
        issue(st.s[J & 3], mt, t + J + 4);                                  \
        __builtin_amdgcn_sched_barrier(0);                                  \
        barrier_after_vmcnt<3 * NL + (((AFTER && J < 2) || (LAST && J == 3)) ? NS : 0)>();
        PS_A(0) PS_A(1) PS_A(2) PS_A(3)
#undef PS_A
      };
      quad(0, std::false_type{}, std::true_type{});
      for (int t = 4; t < nk - 4; t += 4) quad(t, std::false_type{}, std::false_type{});
      quad(nk - 4, std::true_type{}, std::false_type{});
    }
  } else {
    barrier_after_vmcnt<2 * NL + NS>();
    for (int mt = mt_begin; mt < mt_end; ++mt) {
      // as for group A; the epilogue comes after the barrier that closes the
      // last MFMA phase of the M tile
      auto quad = [&](int t, auto last_c, auto after_c) {
        constexpr bool LAST = decltype(last_c)::value;
        constexpr bool AFTER = decltype(after_c)::value;
#define PS_B(J)                                                             \
        e.read_all(0, st.s[J & 3]);                                         \
        issue(st.s[(J + 3) & 3], mt, t + J + 3);                            \
        __builtin_amdgcn_sched_barrier(0);                                  \
        barrier_after_vmcnt<2 * NL + ((AFTER && J < 2) ? NS : 0)>();        \
        mma_all();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                  \
        barrier_after_vmcnt<2 * NL + ((AFTER && J < 2) ? NS : 0)>();        \
        if constexpr (LAST && J == 3) {                                     \
          epi(acc, mt * C::BM);                                             \
          zero_acc(acc);                                                    \
          __builtin_amdgcn_sched_barrier(0);                                \
        }
        PS_B(0) PS_B(1) PS_B(2) PS_B(3)
#undef PS_B
      };
      quad(0, std::false_type{}, std::true_type{});
      for (int t = 4; t < nk - 4; t += 4) quad(t, std::false_type{}, std::false_type{});
      quad(nk - 4, std::true_type{}, std::false_type{});
    }
  }
  barrier_after_vmcnt<0>();
}

// bf16 tiles take the DMA pipeline over the four stages: the ping-pong loop
// when A is K-major, the rolling one when A is M-major (its fragment reads
// transpose both operands, and the longer memory phase then outlasts the
// other group's MFMAs).  fp32 tiles take the register-staged pipeline over
// stage 0 (which is large enough for both of its LDS buffers).
template <class C, bool A_KMAJOR, bool B_KMAJOR, bool KFULL = false>
__device__ __forceinline__ void gemm_any(Acc<C>& acc, const Opnd<typename C::Elem>& A,
                                         const Opnd<typename C::Elem>& B, int m0, int n0, int K,
                                         const DmaStages& st, int tid) {
  if constexpr (sizeof(typename C::Elem) == 2) {
    if constexpr (A_KMAJOR)
      gemm_tile_pp<C, A_KMAJOR, B_KMAJOR, KFULL>(acc, A, B, m0, n0, K, st, tid);
    else
      gemm_tile_dma<C, A_KMAJOR, B_KMAJOR, KFULL>(acc, A, B, m0, n0, K, st, tid);
  } else {
    typedef typename C::Elem T;
    static_assert(C::STAGE * sizeof(T) <= 32768, "an fp32 stage fits one DMA stage");
    gemm_tile<C, A_KMAJOR, B_KMAJOR>(acc, A, B, m0, n0, K, reinterpret_cast<T*>(st.s[0]),
                                     reinterpret_cast<T*>(st.s[1]), tid);
  }
}

// ------------------------------------------------------------- tile order
// Workgroups are dealt to the 8 XCDs round-robin by linear id.  Renumber so
// that ids running together on one XCD are consecutive, then walk tiles in
// groups of `gm` rows so those neighbours share A and B tiles in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  const int q = G / kNumXCDs, r = G % kNumXCDs;
  const int xcd = w % kNumXCDs, slot = w / kNumXCDs;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ void grouped_tile(int l, int TM, int TN, int gm, int& tm, int& tn) {
  const int per = gm * TN;
  const int first = (l / per) * gm;
  const int gs = min(TM - first, gm);
  const int r = l % per;
  tm = first + r % gs;
  tn = r / gs;
}

}  // namespace fce
