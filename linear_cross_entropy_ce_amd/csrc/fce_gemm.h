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
//   32x32 MFMA accumulator layout (wave64): element i of lane l holds
//   row 8*(i/4) + 4*(l/32) + (i%4), column l%32 of the 32x32 block.
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

// bf16: one v_mfma_f32_32x32x16_bf16 per 16-deep K step.  Lane l supplies
// row l%32 and the 8 consecutive k at 8*(l/32) of that step, for A and B
// alike, so the hardware's own k order inside the instruction is irrelevant.
template <>
struct Traits<bf16> {
  static constexpr int VEC = 8;  // elements per 16-byte vector
  typedef bf16x8 Frag;
  // row: LDS row base; x: (first chunk of the fragment) ^ swz(row), in bytes / 16
  __device__ __forceinline__ static Frag frag(const char* row, int x) {
    return *reinterpret_cast<const bf16x8*>(row + (x << 4));
  }
  __device__ __forceinline__ static void mma(floatx16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// fp32: eight v_mfma_f32_32x32x2_f32 per 16-deep K step.  Instruction j
// takes k = 8*(l/32) + j from lane l, so the same 8 consecutive elements per
// lane as the bf16 path are read from LDS.
template <>
struct Traits<float> {
  static constexpr int VEC = 4;
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
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_ELEMS = 2 * STAGE;
  static_assert(BK % 16 == 0 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n),
                                           0x00020000);
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
  floatx16 v[C::FM][C::FN];
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
      for (int i = 0; i < 16; ++i) acc.v[fm][fn][i] = 0.0f;
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
//                     chunk c of row r at chunk c ^ ((r >> 2) & 3).
//   MN-major operand: [32][ROWS] bf16, untransposed rows of k; 16-byte chunk c
//                     of row k at chunk c ^ 4 (k % 4).
// Fragment reads: K-major with ds_read_b128; MN-major with two
// ds_read_b64_tr_b16, whose 16-lane transpose hands lane l the 8 consecutive
// k of column l % 32 (the same fragment a K-major read gives).  With 64 banks
// of 4 bytes, the swizzles put the 16 lanes of a b128 phase (16 consecutive
// rows) and the 32 lanes of a b64 phase (4 k-rows x 32 contiguous bytes x 2
// column groups) on distinct banks.
// Pipeline: STAGES LDS stages; the loads of tile t+STAGES-1 are issued at the
// start of tile t, so each tile's data has STAGES-2 tiles of MFMA work to
// land before the barrier that publishes it.

template <int ROWS, bool KMAJOR, int NT_>
struct DmaOperand;

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

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
    const int c = (tid & 3) ^ ((row >> 2) & 3);
    kc = c * 8;
    tile = op.p + static_cast<int64_t>(mn0) * op.ld;
    rows_left = op.mn_ext - mn0;
    voff0 = static_cast<uint32_t>((row * op.ld + kc) * 2);
    istep = static_cast<uint32_t>(ROWS_PER_I * op.ld * 2);
  }
  __device__ __forceinline__ void load(char* stage, int wave, const Opnd<bf16>& op, int k0,
                                       bool live) const {
    load_rows(stage, wave, op, tile, rows_left, k0, live);
  }
  // The same load for the tile whose first row is mn0 (any tile of `op`).
  __device__ __forceinline__ void load_at(char* stage, int wave, const Opnd<bf16>& op, int mn0,
                                          int k0, bool live) const {
    load_rows(stage, wave, op, op.p + static_cast<int64_t>(mn0) * op.ld, op.mn_ext - mn0, k0,
              live);
  }
  __device__ __forceinline__ void load_rows(char* stage, int wave, const Opnd<bf16>& op,
                                            const bf16* tile_, int64_t rows_left_, int k0,
                                            bool live) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile_ + k0, (rows_left_ * op.ld - k0) * 2);
    const uint32_t off = (live && k0 + kc < op.k_ext) ? voff0 : kOOB;
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
  static_assert(ROWB % 1024 == 0 || 1024 % ROWB == 0, "k-rows tile the 1 KiB DMA blocks");
  static_assert(NI >= 1 && BYTES % (NT * 16) == 0, "MN-major DMA geometry");
  const bf16* tile;
  int mn0;
  uint32_t voff0, istep;

  __device__ __forceinline__ void init(const Opnd<bf16>& op, int mn0_, int tid) {
    mn0 = mn0_;
    const int krow = (tid * 16) / ROWB;
    const int pchunk = ((tid * 16) % ROWB) / 16;
    const int c = pchunk ^ (4 * (krow & 3));
    tile = op.p + mn0;
    voff0 = static_cast<uint32_t>((krow * op.ld + c * 8) * 2);
    istep = static_cast<uint32_t>(KROWS_PER_I * op.ld * 2);
  }
  __device__ __forceinline__ void load(char* stage, int wave, const Opnd<bf16>& op, int k0,
                                       bool live) const {
    // rows k >= k_ext lie past the record count and read as zero
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(tile + static_cast<int64_t>(k0) * op.ld,
                  live ? ((op.k_ext - k0) * op.ld - mn0) * static_cast<int64_t>(2) : 0);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_ptr_t)(stage + i * NT * 16 + wave * 1024), 16, voff0 + i * istep, 0, 0, 0);
  }
};

// Per-lane fragment addressing of one operand (relative to the stage base).
template <int ROWS, bool KMAJOR, int NF>
struct FragAddr;

template <int ROWS, int NF>
struct FragAddr<ROWS, true, NF> {
  int off[2];  // byte offset of fragment 0 for sub-steps 0 and 1
  __device__ __forceinline__ void init(int wave_base, int lane) {
    const int r = wave_base + (lane & 31);
    const int x = (lane >> 5) ^ ((r >> 2) & 3);
    off[0] = r * 64 + 16 * x;
    off[1] = r * 64 + 16 * (x ^ 2);
  }
  __device__ __forceinline__ bf16x8 read(const char* stage, int f, int k16) const {
    return *reinterpret_cast<const bf16x8*>(stage + off[k16] + f * 32 * 64);
  }
};

template <int ROWS, int NF>
struct FragAddr<ROWS, false, NF> {
  static constexpr int ROWB = ROWS * 2;
  int off[NF];  // byte offset for fragments f = 0..NF-1 (sub-step 0, half 0)
  __device__ __forceinline__ void init(int wave_base, int lane) {
    const int gq = lane >> 4, a = lane & 15;
    const int kr0 = 8 * (gq >> 1) + (a >> 2);
    const int g = 4 * (a >> 2);  // swizzle of row kr0 + 4h + 16 k16 (all = kr0 mod 4)
    const int mnoff = 16 * (gq & 1) + 4 * (a & 3);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int mn = wave_base + 32 * f + mnoff;
      off[f] = kr0 * ROWB + 16 * ((mn >> 3) ^ g) + (mn & 7) * 2;
    }
  }
  __device__ __forceinline__ bf16x8 read(const char* stage, int f, int k16) const {
    const char* p = stage + off[f] + k16 * 16 * ROWB;
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
// operand DMA, fragment reads, MFMAs and the pinned interleaving of one
// 32-deep K step.  Any wave layout C::WAVES_M x C::WAVES_N whose wave tile is
// a multiple of 32 x 32; 256 or 512 threads.
template <class C, bool A_KMAJOR, bool B_KMAJOR>
struct DmaEngine {
  static constexpr int S = 4, BK = 32;
  static constexpr int B_OFF = C::BM * BK * 2;
  static constexpr int FM = C::FM, FN = C::FN;
  typedef DmaOperand<C::BM, A_KMAJOR, C::NT> DA;
  typedef DmaOperand<C::BN, B_KMAJOR, C::NT> DB;
  static constexpr int NL = DA::NI + DB::NI;  // DMA instructions per thread per K tile
  // LDS read instructions per fragment set: one b128 per K-major fragment,
  // two b64 transpose reads per MN-major fragment
  static constexpr int NR = FM * (A_KMAJOR ? 1 : 2) + FN * (B_KMAJOR ? 1 : 2);
  static constexpr int NMMA = FM * FN;         // MFMAs per 16-deep sub-step
  static constexpr int NG = NMMA / 2;          // interleave groups (first half of the MFMAs)
  static constexpr int RG = (NR + NG - 1) / NG, LG = (NL + NG - 1) / NG;
  static_assert(C::BM * BK * 2 + C::BN * BK * 2 <= 32768, "one K tile per 32 KiB stage");

  DA da;
  DB db;
  FragAddr<C::BM, A_KMAJOR, FM> fa_addr;
  FragAddr<C::BN, B_KMAJOR, FN> fb_addr;
  bf16x8 fa[2][FM], fb[2][FN];
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
  __device__ __forceinline__ void read(int set, const char* stage, int k16) {
#pragma unroll
    for (int f = 0; f < (FM > FN ? FM : FN); ++f) {
      if (f < FM) fa[set][f] = fa_addr.read(stage, f, k16);
      if (f < FN) fb[set][f] = fb_addr.read(stage + B_OFF, f, k16);
    }
  }
  __device__ __forceinline__ void mma(Acc<C>& acc, int set) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc.v[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][fm], fb[set][fn],
                                                                acc.v[fm][fn], 0, 0, 0);
  }
  // Pin the order: the reads of the next fragment set (and the DMA issue)
  // go between the first half of the current set's MFMAs, so both fragment
  // sets stay live and no MFMA waits on an LDS round trip.
  __device__ __forceinline__ static void pin(bool with_dma) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, RG, 0);
      if (with_dma) __builtin_amdgcn_sched_group_barrier(kSchedVMEMRead, LG, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMFMA, NMMA - NG, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // One K tile in stage `cur`: prefetch (issue_next) into the stage of the
  // previous tile (free since the previous barrier), read sub-step 1, MFMA
  // sub-step 0, publish the next tile (wait for this thread's DMA of it,
  // barrier), read its sub-step 0, MFMA sub-step 1.
  template <class Issue>
  __device__ __forceinline__ void step(Acc<C>& acc, const char* cur, const char* nxt,
                                       Issue&& issue_next) {
    issue_next();
    read(1, cur, 1);
    mma(acc, 0);
    pin(true);
    barrier_after_vmcnt<NL * (S - 2)>();
    read(0, nxt, 0);
    mma(acc, 1);
    pin(false);
  }
};

template <class C>
__device__ __forceinline__ void zero_acc(Acc<C>& acc) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc.v[fm][fn][i] = 0.0f;
}

// One BM x BN bf16 output tile, operands in any layout, through the 4-stage
// DMA pipeline.  The K loop is unrolled by the stage count so every stage
// reference is static.  When the tile count is not a multiple of four the
// last trip runs on tiles past the end, whose stages hold the zeros of
// out-of-range loads: their MFMAs add exact zeros.  Ends with all DMA
// drained and a barrier, so the stages may be reused after it.
template <class C, bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void gemm_tile_dma(Acc<C>& acc, const Opnd<bf16>& A,
                                              const Opnd<bf16>& B, int m0, int n0, int K,
                                              const DmaStages& st, int tid) {
  typedef DmaEngine<C, A_KMAJOR, B_KMAJOR> E;
  constexpr int S = E::S, BK = E::BK;
  zero_acc(acc);
  const int nk = (K + BK - 1) / BK;
  if (nk <= 0) return;
  E e;
  e.init(A, B, m0, n0, tid);
  auto issue = [&](char* stage, int kt) {
    const bool live = kt < nk;
    e.da.load(stage, e.wave, A, kt * BK, live);
    e.db.load(stage + E::B_OFF, e.wave, B, kt * BK, live);
  };
  issue(st.s[0], 0);
  issue(st.s[1], 1);
  issue(st.s[2], 2);
  barrier_after_vmcnt<E::NL * (S - 2)>();
  e.read(0, st.s[0], 0);
  for (int kt = 0; kt < nk; kt += S) {
    e.step(acc, st.s[0], st.s[1], [&] { issue(st.s[3], kt + 3); });
    e.step(acc, st.s[1], st.s[2], [&] { issue(st.s[0], kt + 4); });
    e.step(acc, st.s[2], st.s[3], [&] { issue(st.s[1], kt + 5); });
    e.step(acc, st.s[3], st.s[0], [&] { issue(st.s[2], kt + 6); });
  }
  // the prefetches past the last tile still write (zeros) into LDS: drain them
  barrier_after_vmcnt<0>();
}

// Consecutive BM-row M tiles mt_begin .. mt_end-1 (K-major A, full K each)
// against one BN-column N tile of K-major B, as ONE stream of K tiles: the
// DMA for the next M tile's first K tiles is issued while the current one
// finishes, so the pipeline never drains between M tiles.  After each M tile
// epi(acc, m0) consumes the accumulators (registers only; LDS stays with the
// pipeline) and they restart from zero.  Needs K % 128 == 0 (M tile
// boundaries on the unrolled-by-four trip).  Ends with all DMA drained and a
// barrier.
template <class C, class Epi>
__device__ __forceinline__ void gemm_stream_dma(const Opnd<bf16>& A, const Opnd<bf16>& B,
                                                int mt_begin, int mt_end, int n0, int K,
                                                const DmaStages& st, int tid, Epi&& epi) {
  typedef DmaEngine<C, true, true> E;
  constexpr int S = E::S, BK = E::BK;
  const int nk = K / BK;
  const int total = (mt_end - mt_begin) * nk;
  Acc<C> acc;
  zero_acc(acc);
  if (total <= 0) return;
  E e;
  e.init(A, B, mt_begin * C::BM, n0, tid);
  // stream position g = (M tile index) * nk + (K tile index)
  auto issue = [&](char* stage, int g) {
    const bool live = g < total;
    const int gg = live ? g : 0;
    const int k0 = (gg % nk) * BK;
    e.da.load_at(stage, e.wave, A, (mt_begin + gg / nk) * C::BM, k0, live);
    e.db.load(stage + E::B_OFF, e.wave, B, k0, live);
  };
  issue(st.s[0], 0);
  issue(st.s[1], 1);
  issue(st.s[2], 2);
  barrier_after_vmcnt<E::NL * (S - 2)>();
  e.read(0, st.s[0], 0);
  for (int mt = mt_begin; mt < mt_end; ++mt) {
    const int base = (mt - mt_begin) * nk;
    for (int kt = 0; kt < nk; kt += S) {
      const int g = base + kt;
      e.step(acc, st.s[0], st.s[1], [&] { issue(st.s[3], g + 3); });
      e.step(acc, st.s[1], st.s[2], [&] { issue(st.s[0], g + 4); });
      e.step(acc, st.s[2], st.s[3], [&] { issue(st.s[1], g + 5); });
      e.step(acc, st.s[3], st.s[0], [&] { issue(st.s[2], g + 6); });
    }
    epi(acc, mt * C::BM);
    zero_acc(acc);
  }
  barrier_after_vmcnt<0>();
}

// bf16 tiles take the DMA pipeline over the four stages, fp32 tiles the
// register-staged one over stage 0 (which is large enough for both of its
// LDS buffers).
template <class C, bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void gemm_any(Acc<C>& acc, const Opnd<typename C::Elem>& A,
                                         const Opnd<typename C::Elem>& B, int m0, int n0, int K,
                                         const DmaStages& st, int tid) {
  if constexpr (sizeof(typename C::Elem) == 2) {
    gemm_tile_dma<C, A_KMAJOR, B_KMAJOR>(acc, A, B, m0, n0, K, st, tid);
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
