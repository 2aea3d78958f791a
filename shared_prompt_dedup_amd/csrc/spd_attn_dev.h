// Device building blocks shared by the bf16 split-attention kernels (gfx950).
//
// Matrix core: v_mfma_f32_32x32x16_bf16 (wave64).  Lane l supplies row
// (l % 32) of A and column (l % 32) of B as 8 bf16 along the contraction; the
// fp32 result holds C[8 (r / 4) + 4 (l / 32) + (r % 4)][l % 32] in register r.
// Only the pairing of A and B contraction slots matters, so an operand may list
// its 8 contraction indices in any order as long as the other operand lists
// the same ones.  A result reused as an operand (probabilities, dS) therefore
// lists, in lane half h, the rows {4h..4h+3, 8+4h..8+4h+3} of each 16-row step.
//
// Tiles live in LDS row-major with 16-byte chunks XOR-swizzled by row: slot =
// chunk ^ f(row).  LDS serves 256 bytes (all 64 banks) per cycle: 16 lanes of a
// 16-byte read, or 32 lanes of an 8-byte read.  f makes both patterns in use
// conflict-free: sixteen consecutive rows read at one chunk land on sixteen
// distinct slots, and a half-wave of transposing reads (4 consecutive rows x
// 4 consecutive chunks, see below) lands on sixteen distinct slots.  The tiles
// are filled with direct-to-LDS loads (global_load_lds_dwordx4: lane l's 16
// bytes land at M0 + 16 l), so no registers or ALU time are spent staging them.
//
// The transposed operands (V^T, K^T, Q^T, dO^T) are read straight from those
// row-major tiles with ds_read_b64_tr_b16: in each 16-lane group, output lane
// i, element j is element (i % 4) of the 8 bytes read by lane 4 j + i / 4.
// If lane s of the group reads row key(s / 4), columns c0 + 4 (s % 4) ... + 3,
// output lane i holds column c0 + i of rows key(0..3): the column-major slice
// an MFMA operand needs, with the 4 rows free to choose.
#pragma once

#include <cstdint>

#include "spd_attn.h"

namespace spd {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

__device__ inline bf16x8 zero8() {
  return __builtin_bit_cast(bf16x8, i16x8{0, 0, 0, 0, 0, 0, 0, 0});
}

__device__ inline bf16x8 ld_global8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ inline bf16x8 ld_lds8(const char *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Two transposing 8-byte LDS reads concatenated into one MFMA operand.
__device__ inline bf16x8 ld_lds_tr_pair(const char *p0, const char *p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p1));
  const i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// p, with the compiler unable to see through the value: per-lane LDS bases
// are then formed once per tile and every constant step folds into the
// instruction's offset field, instead of one precomputed sum being kept live
// per (base, step) pair across the loop.
__device__ inline const char *opaque_lds(const char *p) {
  auto q = (const __attribute__((address_space(3))) char *)(p);
  asm volatile("" : "+v"(q));
  return (const char *)(q);
}

// Row (0..31) of register r of a 32x32 result for lane half h.
__device__ inline int c_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Row swizzle.  256-byte rows (D = 128): f(r) = 4 (r % 4) + (r / 4) % 4, a
// permutation of the 16 slots over 16 rows, whose four rows of an aligned
// quad differ in the top two slot bits.  128-byte rows (D = 64, two rows per
// bank cycle): f(r) = 4 ((r / 2) % 2) + (r / 4) % 4, a permutation of the 8
// slots over the 8 rows of either parity, whose same-parity rows of a quad
// differ in slot bit 2.
template <int D>
__device__ inline int swz_of(int row) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a swizzled tile of D columns.
template <int D>
__device__ inline int swz_off(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ swz_of<D>(row)) << 4);
}

// One direct-to-LDS load: lane l's 16 bytes at base + voff land at LDS
// address lds + 16 l (lds wave-uniform, base a wave-uniform 64-bit address
// held in SGPRs, voff a per-lane 32-bit byte offset).  It is issued from
// inline assembly: the compiler, seeing an LDS DMA, would otherwise make every
// later transposing LDS read wait for all outstanding vector loads, including
// the prefetches of later stages.  Callers wait for completion themselves
// (wait_ring) before a barrier publishes the data.
//
// The compiler does not know that the assembly holds a vector-memory load, so
// it pads none of that load's wait states.  A vector-memory instruction must
// come at least 5 wait states after a VALU write of an SGPR it reads, and the
// compiler may produce base or M0 with one (v_readlane when it reloads a
// spilled SGPR, v_readfirstlane): the load would then read a stale address.
// The assembly therefore copies both with scalar moves, whose reads of a
// VALU-written SGPR are interlocked and whose results a load may read at once;
// the s_nop is the one wait state an LDS DMA needs after M0 is written.
__device__ inline void dma16(const void *base, unsigned voff, const char *lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_void *)(lds))));
  const void *b;
  unsigned m0;   // M0 is an output of the assembly, not a clobber: the compiler knows it is written
  asm volatile("s_mov_b64 %0, %3\n\ts_mov_b32 %1, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %0"
               : "=&s"(b), "=&{m0}"(m0)
               : "v"(voff), "s"(base), "s"(m)
               : "memory");
}

// Direct-to-LDS copy of rows [r0, r0 + ROWS) of a [*, H, D] bf16 tensor (head
// hh) into a swizzled tile, spread over NW waves.  Rows past T - 1 are clamped
// to T - 1: they hold real (finite) data and every consumer masks them.
template <int ROWS, int D, int NW>
__device__ inline void dma_rows(char *tile, const __bf16 *src, int r0, int T, int H, int hh, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int CHUNKS = ROWS * CPR;
  static_assert(CHUNKS % (NW * 64) == 0, "tile must split into whole wave loads");
  constexpr int PER_WAVE = CHUNKS / (NW * 64);
  const int rb = min(r0, T - 1);       // base row; rows rb + r, r <= rmax, stay below T
  const int rmax = T - 1 - rb;
  const __bf16 *base = src + (int64_t(rb) * H + hh) * D;
  const unsigned row_bytes = static_cast<unsigned>(H) * D * 2;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int blk = wave * PER_WAVE + i;
    const int L = blk * 64 + lane;
    const int r = L / CPR;
    const int slot = L % CPR;
    const int chunk = slot ^ swz_of<D>(r);
    const unsigned voff = static_cast<unsigned>(min(r, rmax)) * row_bytes + (chunk << 4);
    dma16(base, voff, tile + blk * 1024);
  }
}

// As dma_rows, for rows x0 .. x0 + ROWS - 1 of a virtual row space joining two
// ranges: virtual row x < lenV is row v0 + x, later ones row u0 + x - lenV
// (rows past T - 1 are clamped to it; the caller masks what it does not own).
// Lane offsets are 32-bit from the head's first row: the entry points
// reject T * Hkv * D * 2 >= 4 GiB before launching.
template <int ROWS, int D, int NW>
__device__ inline void dma_rows2(char *tile, const __bf16 *src, int x0, int lenV, int v0, int u0, int T, int H,
                                 int hh, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int CHUNKS = ROWS * CPR;
  static_assert(CHUNKS % (NW * 64) == 0, "tile must split into whole wave loads");
  constexpr int PER_WAVE = CHUNKS / (NW * 64);
  const __bf16 *base = src + int64_t(hh) * D;
  const unsigned row_bytes = static_cast<unsigned>(H) * D * 2;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int blk = wave * PER_WAVE + i;
    const int L = blk * 64 + lane;
    const int r = L / CPR;
    const int slot = L % CPR;
    const int chunk = slot ^ swz_of<D>(r);
    const int x = x0 + r;
    const int row = min(x < lenV ? v0 + x : u0 + (x - lenV), T - 1);
    dma16(base, static_cast<unsigned>(row) * row_bytes + (chunk << 4), tile + blk * 1024);
  }
}

// s_waitcnt immediate that waits only until at most N vector-memory operations
// of this wave are outstanding (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] in [15:14]).
template <int N>
struct VmCnt {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  static constexpr int imm = (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14);
};

// Waits for every outstanding vector-memory load of this wave.  Called after a
// kernel's own register loads and before its first direct-to-LDS load: the
// compiler cannot count the assembly-issued loads, so a register load it still
// believed pending would make it wait for every load in flight, prefetches
// included, at each use.
__device__ inline void wait_vm_all() { __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm); }

// Ring wait for tile i of n when the ring keeps up to STAGES tiles in flight
// and each tile costs PER direct-to-LDS loads per wave: tiles i+1 .. i+STAGES-2
// may still be loading.  Then a block barrier.
template <int STAGES, int PER>
__device__ inline void wait_ring(int i, int n) {
  if (i + STAGES - 2 < n)
    __builtin_amdgcn_s_waitcnt(VmCnt<(STAGES - 2) * PER>::imm);
  else
    __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Marks a wave-uniform branch as worth keeping: the compiler may not
// speculate a volatile asm, so the guarded work (e.g. masking) runs only when
// the condition holds instead of being turned into selects on every pass.
__device__ inline void keep_branch() { asm volatile(""); }

// Sets this wave's issue priority, pinned in place: no instruction is
// scheduled across the change.
template <int P>
__device__ inline void set_prio() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(P);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Instruction classes of the scheduler's group barriers.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Orders the scheduling region it ends: N matrix-core instructions, each
// with R LDS operand reads, the reads issued A MFMAs ahead of their use (the
// compiler otherwise waits on each read right before its MFMA).
template <int A, int N, int R>
__device__ inline void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, A * R, 0);
#pragma unroll
  for (int j = 0; j < N - A; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, A, 0);
}

}  // namespace dev
}  // namespace spd
