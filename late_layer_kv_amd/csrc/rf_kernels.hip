// HIP kernels of the late-layer cache fill for gfx950 (MI355X).
//
// Two bf16 MFMA contractions carry the work ("RidgeFill: Training-Free
// Late-Layer Cache Fill for Faster Prefill", sections 2.1-2.2):
//   map_gemm : Y_l = X_F A_l^T + b_l for a group of late layers, the rows of
//              X gathered through the fill-row index on the way into LDS;
//   kv_gemm  : K|V = (Y_l W'^T) / rms(Y_l) with W' = [W_k|W_v] * gamma, then
//              RoPE on the key columns and a bf16 scatter into each layer's
//              cache slot for the row.
//
// Both use one main loop.  A workgroup of 4 waves owns a 256x256 output tile
// (256 output features x 256 rows); each wave owns 128 features x 128 rows as
// 8x8 blocks of v_mfma_f32_16x16x32_bf16.  The weight matrix is the MFMA "A"
// operand and the data rows the "B" operand, so in the accumulator every lane
// holds whole data rows: lane l owns row (l & 15) of each 16-row block and
// features 4 (l >> 4) .. + 3 of each 16-feature block.  The RoPE partner of a
// key feature therefore sits in the same lane and register; a row's norm and
// QK-norm sums reduce over the four lanes l, l ^ 16, l ^ 32, l ^ 48.
//
// Why 16x16x32 rather than 32x32x16: both issue the same flops per cycle,
// but the part runs power-limited at full MFMA load and the 32x32 form draws
// more per flop (it moves four times the accumulator data per instruction).
// In a register-only loop on random bf16 data the 16x16 form held 2.07 GHz
// and 2.04 PFLOP/s against 1.83 GHz and 1.81 PFLOP/s for the 32x32 form; in
// these kernels the switch gained 7-10%.  The MFMAs are inline assembly (see
// mfma16) so their accumulators stay in place.
//
// Operand tiles stream global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
// staging; see OpSrc) in stages of 64 contraction columns, so every operand row of a
// stage is one full 128-byte line (one L2 request per row per stage; 32-column
// stages fetched half lines and cost the texture path about 14% of the map
// contraction's speed).  The 160 KB of LDS is a ring of five 32 KB slots, each
// holding one operand (256 rows x 128 bytes) of one stage, so about one and a
// half stages of loads are in flight while one is consumed.  Within a stage
// the MFMA operand fragments of the next 32-column step are read into a
// second register set while the current step's MFMAs run.  The one
// workgroup barrier per stage sits between the two steps; it is issued
// without a memory fence (the fence would make every wave wait for all
// in-flight prefetches).  Each wave instead waits (vmcnt) for its own loads
// of the next stage only; the barrier then publishes them and frees the two
// slots just consumed.
//
// LDS slot rows are 128 bytes (64 bf16).  gfx950's LDS has 64 banks (256
// bytes per cycle, 16 lanes of a 16-byte read per pass), so the 16-byte chunk c
// of row r is stored at chunk position c ^ ((r >> 1) & 7): the 16 rows one
// pass reads then cover all 64 banks.  The epilogue reuses the LDS as a
// 256x256 bf16 staging tile so that every global store is a 16-byte,
// row-contiguous write.
//
// Reduction order is fixed by the tile shape alone (no split-K, no atomics on
// values), so results are bitwise reproducible and independent of which other
// rows share a tile and of how many layers share a launch.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rf_internal.h"

namespace rf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_ptr_t;
typedef const __attribute__((address_space(1))) void gbl_ptr_t;

constexpr int kThreads = 256;
constexpr int kBK = 64;                               // contraction columns per stage
constexpr int kRing = 5;                              // LDS slots, one operand of one stage each
constexpr int kRowBytes = kBK * 2;                    // 128 B per slot row
constexpr int kSlotBytes = 256 * kRowBytes;           // 32 KB
constexpr int kLoadsPerSlot = 8;                      // LDS-DMA loads per wave per slot
constexpr int kStageRowBytes = kTileN * 2;            // 512 B per staged output row
constexpr int kStagingBytes = kTileM * kStageRowBytes;  // 128 KB
constexpr int kSlotOffset = kStagingBytes;            // 256 int32 slot ids after the staging tile
constexpr int kLdsBytes = (kRing * kSlotBytes > kStagingBytes + 1024) ? kRing * kSlotBytes : kStagingBytes + 1024;
static_assert(kTileK % kBK == 0, "host contraction granule must be a multiple of the stage depth");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of gfx950");

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 pair, packed (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Row sums of squares for the norm are formed the same way wherever the row
// comes from (map epilogue or a pass over given inputs), so that the two give
// bitwise-equal factors: per 256-feature tile, each of its two 128-feature
// halves is split into four lane parts (features 16 nb + 4 q + v), each part
// summed over nb = 0..7 with this pair of bf16 dot products (4 consecutive
// features packed as two bf16 pairs), then (q0 + q1) + (q2 + q3), then
// half 0 + half 1; tiles are added in ascending order.
__device__ __forceinline__ float sq4(float s, uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_bit_cast(bf16x2, lo), b = __builtin_bit_cast(bf16x2, hi);
  s = __builtin_amdgcn_fdot2_f32_bf16(a, a, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(b, b, s, false);
}

// RoPE of one (j, j + hd/2) pair of already-scaled values.  The fused form is
// spelled out: left to contract x1 c - x2 s itself, the compiler may keep
// either product rounded, and its choice differed between call sites.  Every
// rotation (key heads, indexer heads in either tile shape) calls this, so a
// key head and an indexer head with the same weights round identically.
__device__ __forceinline__ void rotate(float x1, float x2, float co, float si, float& y1, float& y2) {
  y1 = __builtin_fmaf(x1, co, -(x2 * si));
  y2 = __builtin_fmaf(x2, co, x1 * si);
}

// Workgroups are dealt round-robin to the 8 XCDs.  Two renumberings, so that
// the 32 workgroups an XCD runs at once are consecutive logical tiles (which
// the tile order below makes share operand strips in that XCD's L2):
//  * contiguous: XCD x works through one contiguous eighth of the tiles (the
//    XCDs are then at different layers and rows of the launch);
//  * chunked: XCD x takes chunks x, x + 8, x + 16, ... of 32 tiles, so the 8
//    XCDs work on neighbouring chunks of the same layer together and the
//    256 MB MALL serves each layer's map and the current row strips to all of
//    them (the map contraction runs 4-5% faster this way; the key/value
//    contraction, whose weights are small, 1% slower).
__device__ __forceinline__ int xcd_remap_contiguous(int bid, int n) {
  const int q = n >> 3, r = n & 7, x = bid & 7, local = bid >> 3;
  return (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

__device__ __forceinline__ int xcd_remap_chunked(int bid, int n) {
  constexpr int kChunk = 32;
  if (bid >= n / (8 * kChunk) * (8 * kChunk)) return bid;  // the last, partial round in dispatch order
  const int x = bid & 7, local = bid >> 3;
  return (local / kChunk) * (8 * kChunk) + x * kChunk + local % kChunk;
}

struct TileCoord {
  int g, tm, tn;
};

// Logical tile -> (layer, row tile, feature tile).  Inside a layer tiles go
// down groups of GM row tiles for one feature tile before moving on, so the
// 32 workgroups an XCD runs at once cover GM row strips x 32/GM weight strips
// (measured best: 4 for both contractions with their remappings above).
template <int GM>
__device__ __forceinline__ TileCoord tile_coord(int t, int tiles_m, int tiles_n) {
  const int per_layer = tiles_m * tiles_n;
  TileCoord c;
  c.g = t / per_layer;
  const int u = t - c.g * per_layer;
  const int per_group = GM * tiles_n;
  const int grp = u / per_group;
  const int first_m = grp * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int v = u - grp * per_group;
  c.tm = first_m + v % gsz;
  c.tn = v / gsz;
  return c;
}

// The same order with the group height chosen at launch (the K/V contraction:
// 4 row tiles when the launch has 8 or fewer feature tiles per layer that
// divide 32, so that an XCD's 32 co-running tiles are whole groups; 2 when
// an indexer head makes it 9, measured 2.5% faster for that launch).
__device__ __forceinline__ TileCoord tile_coord_rt(int t, int tiles_m, int tiles_n, int gm) {
  const int per_layer = tiles_m * tiles_n;
  TileCoord c;
  c.g = t / per_layer;
  const int u = t - c.g * per_layer;
  const int per_group = gm * tiles_n;
  const int grp = u / per_group;
  const int first_m = grp * gm;
  const int gsz = min(tiles_m - first_m, gm);
  const int v = u - grp * per_group;
  c.tm = first_m + v % gsz;
  c.tn = v / gsz;
  return c;
}

// Wait until at most `slots` slots of this wave's loads are still in flight
// (loads complete in issue order for the vmcnt counter).
__device__ __forceinline__ void wait_slots(int slots) {
  switch (slots) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
  }
}
static_assert(kLoadsPerSlot == 8, "wait_slots immediates assume 8 loads per slot");

// Workgroup barrier without a memory fence (see the file comment).  The
// "memory" clobber keeps the compiler from moving LDS accesses across it; the
// hardware ordering the loop relies on is stated where it is used.  The
// wave's own LDS reads have returned before it arrives (lgkmcnt(0)), so a slot
// it read before the barrier may be refilled by any wave after it; the reads
// were issued most of a step earlier, so the wait costs nothing.
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS position of 16-byte chunk c (0..7) of slot row r.
__device__ __forceinline__ int slot_pos(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 7)) << 4); }

// Where one operand of the main loop is read: for load instruction j, this
// lane's 16-byte chunk of column block 0 (see load_chunk); stage t adds
// t * 128 bytes.  Usually (OpSrc<false>) the operand is one raw buffer
// resource with 32-bit byte offsets per lane, and the stage offset goes in the
// instruction's scalar offset (buffer_load_dwordx4 ... lds): 16 fewer VGPRs
// than 64-bit pointers and no per-load address arithmetic; measured 0.7%
// faster on the whole fill.  An operand that spans 4 GiB or more
// (OpSrc<true>) keeps 64-bit pointers and global_load_lds.
template <bool WIDE>
struct OpSrc;
template <>
struct OpSrc<false> {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off[8];
  __device__ void init(const void* base, size_t bytes) {
    // bytes < 4 GiB here: every offset plus the stage offset stays below it
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                          static_cast<int>(static_cast<uint32_t>(bytes)), 0x00020000);
  }
  __device__ void set(int j, size_t byte_off) { off[j] = static_cast<uint32_t>(byte_off); }
  __device__ __forceinline__ void load(int j, size_t kbyte, char* dst) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t*)dst, 16, off[j], static_cast<int>(kbyte), 0, 0);
  }
};
template <>
struct OpSrc<true> {
  const char* p[8];
  const char* base_;
  __device__ void init(const void* base, size_t) { base_ = static_cast<const char*>(base); }
  __device__ void set(int j, size_t byte_off) { p[j] = base_ + byte_off; }
  __device__ __forceinline__ void load(int j, size_t kbyte, char* dst) const {
    __builtin_amdgcn_global_load_lds((gbl_ptr_t*)(p[j] + kbyte), (lds_ptr_t*)dst, 16, 0, 0);
  }
};

// The 8 loads of one slot (one operand of one stage) for this wave:
// instruction j covers slot rows 64 w + 8 j .. + 7 and lane i lands at LDS byte
// 1 KB * (8 w + j) + 16 i, i.e. row 64 w + 8 j + i / 8, position i % 8.
template <class Src>
__device__ __forceinline__ void issue_slot(const Src& src, size_t kbyte, char* dst) {
#pragma unroll
  for (int j = 0; j < kLoadsPerSlot; ++j) src.load(j, kbyte, dst + j * 1024);
}

// Column chunk a lane fetches for instruction j: position i % 8 of row
// 64 w + 8 j + i / 8 holds chunk (i % 8) ^ ((row >> 1) & 7).  The 8 lanes of a
// row fetch its 8 chunks, one whole 128-byte line.
__device__ __forceinline__ int load_chunk(int lane, int j) { return (lane & 7) ^ ((4 * j + (lane >> 4)) & 7); }

__device__ __forceinline__ int ring(int s) { return s >= kRing ? s - kRing : s; }

// A 16-byte store marked non-temporal: Y and the caches are not read again
// within a launch, and keeping them out of the L2 and the MALL leaves that
// room to the maps and rows the contractions re-read (on one box the step ran
// 1.5% faster with it, on another it tied; never slower).
__device__ __forceinline__ void store16_nt(void* dst, const uint4& v) {
  __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&v), static_cast<u32x4*>(dst));
}

// ---- Main loop -----------------------------------------------------------
// The wave's 128x128 block is 8x8 blocks of v_mfma_f32_16x16x32_bf16: a lane
// owns row (l & 15) of each 16-row block and features 4 (l >> 4) .. + 3 of
// each 16-feature block.  A 64-column stage is two 32-column steps; the
// fragments of the next step are read into the second register set while the
// current step's 64 MFMAs run.
struct Frags {
  bf16x8 a[8], b[8];
};

// MFMA i of a 32-column step works on block (i / 8, mfma_col(i)): the 8x8
// blocks in serpentine order, so consecutive MFMAs always share an operand
// fragment (the A fragment along a row, the B fragment at each turn).  Taking
// the rows left to right every time instead ran both contractions 0.4-0.5%
// slower (bitwise the same results; interleaved runs on one box).
__device__ __forceinline__ constexpr int mfma_col(int i) { return ((i >> 3) & 1) ? 7 - (i & 7) : (i & 7); }

__device__ __forceinline__ void read_frags(Frags& f, const char* ws, const char* xs, int aoff, int boff) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(ws + aoff + i * 16 * kRowBytes);
#pragma unroll
  for (int i = 0; i < 8; ++i) f.b[i] = *reinterpret_cast<const bf16x8*>(xs + boff + i * 16 * kRowBytes);
}

// One MFMA 16x16x32 accumulating in place.  Written as inline assembly: the
// compiler's register allocation of the builtin copies accumulators between
// AGPRs around every instruction at this block count.  The statement is
// volatile, so memory operations keep their place relative to it and the
// fragment reads / operand loads below interleave exactly as written.
__device__ __forceinline__ void mfma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// The first MFMA into an accumulator: the addend is the inline constant 0,
// so the accumulators are never written by vector instructions before the
// MFMA chain (no zeroing, and no wait states between such writes and the
// first MFMA that reads them).
__device__ __forceinline__ void mfma16_first(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

// One accumulator value read out of its AGPR where it is used.  The compiler
// otherwise copies all 256 accumulators into VGPRs at the end of the main
// loop, which leaves the epilogue no registers for its loads.
__device__ __forceinline__ float agpr(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// The 64 MFMAs of one 32-column step on fragments f.  With READ, the 16
// fragment reads of the next step (into nf, from slots ws / xs) follow MFMAs
// 0..15 one each; with LOAD, the 8 operand loads of one slot follow MFMAs
// 16, 22, ..., 58.  Spread over the step, the 32 loads a workgroup issues per
// step reach the texture path at about a third of the rate they do bunched
// after every second MFMA, and the waves' instruction streams stall less
// behind a full load queue (both contractions ran 1-2% faster).
// With FIRST (the first step of a tile), every MFMA starts its accumulator
// from 0 (each of the 64 blocks is met exactly once per step).  A fragment
// register is refilled at least 8 MFMA issues after the last MFMA that read
// it: A fragment n is last read by MFMA 8n+7 and refilled after MFMA n of the
// next step, B fragment m last read by MFMA 63-m (the last row of blocks runs
// right to left) and refilled after MFMA 8+m.
template <bool READ, bool LOAD, bool FIRST = false, class Src>
__device__ __forceinline__ void mma_step(const Frags& f, f32x4 (&acc)[8][8], Frags& nf, const char* ws,
                                           const char* xs, int aoff, int boff, const Src& src,
                                           size_t kbyte, char* dst) {
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const int nb = i >> 3, mb = mfma_col(i);
    if (FIRST)
      mfma16_first(acc[nb][mb], f.a[nb], f.b[mb]);
    else
      mfma16(acc[nb][mb], f.a[nb], f.b[mb]);
    if (READ && i < 8) nf.a[i] = *reinterpret_cast<const bf16x8*>(ws + aoff + i * 16 * kRowBytes);
    if (READ && i >= 8 && i < 16) nf.b[i - 8] = *reinterpret_cast<const bf16x8*>(xs + boff + (i - 8) * 16 * kRowBytes);
    if (LOAD && i >= 16 && (i - 16) % 6 == 0 && i <= 58) {
      const int j = (i - 16) / 6;
      src.load(j, kbyte, dst + j * 1024);
    }
  }
}

// One stage t on slots sw (weights) and sw + 1 (data rows), ending with stage
// t+1 published.  Slot sequence number u = 0, 1, 2, ... is the weights of
// stage u / 2 (even u) or its data rows (odd u), in ring slot u % 5.
//   PEND : during step 0, load u = 2t+4 (weights of stage t+2) into slot
//          sw + 4, free since the barrier that opened stage t;
//   ISSUE: during step 1, after the barrier, load u = 2t+5 (data rows of
//          stage t+2) into slot sw, free once every wave has passed it;
//   WAIT : slots this wave may still have in flight at the barrier (stage t+1
//          needs u <= 2t+3 landed; u = 2t+4 may still fly).
// Step 0 reads step 1's fragments from the current slots; after the barrier,
// step 1 reads the next stage's step-0 fragments.
template <bool PEND, bool ISSUE, int WAIT, bool FIRST = false, class Src>
__device__ __forceinline__ void stage(Frags& fa, Frags& fb, f32x4 (&acc)[8][8], int& sw, int t,
                                        char* smem, char* mydst, const Src& wsrc, const Src& xsrc,
                                        const int (&aoff)[2], const int (&boff)[2]) {
  const char* ws = smem + sw * kSlotBytes;
  const char* xs = smem + ring(sw + 1) * kSlotBytes;
  mma_step<true, PEND, FIRST>(fa, acc, fb, ws, xs, aoff[1], boff[1], wsrc, static_cast<size_t>(t + 2) * kRowBytes,
                                mydst + ring(sw + 4) * kSlotBytes);
  wait_slots(WAIT);
  barrier();
  const int nsw = ring(sw + 2);
  mma_step<true, ISSUE>(fb, acc, fa, smem + nsw * kSlotBytes, smem + ring(nsw + 1) * kSlotBytes, aoff[0], boff[0],
                          xsrc, static_cast<size_t>(t + 2) * kRowBytes, mydst + sw * kSlotBytes);
  sw = nsw;
}

// Main loop over nk stages, shared by both contractions.  On return acc[nb][mb]
// holds features 16 nb + 4 (l >> 4) + v, row 16 mb + (l & 15) of the wave's block.
template <class Src>
__device__ __forceinline__ void mainloop(const Src& wsrc, const Src& xsrc, int nk, char* smem, f32x4 (&acc)[8][8]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int r15 = lane & 15, q = lane >> 4;
  char* const mydst = smem + wave * kLoadsPerSlot * 1024;
  // Row r of a 16-row block is lane & 15, its chunk for step s is 4 s + q;
  // 16-row blocks are 2 KB apart and share the chunk permutation.
  int aoff[2], boff[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    aoff[st] = slot_pos(wn * 128 + r15, 4 * st + q);
    boff[st] = slot_pos(wm * 128 + r15, 4 * st + q);
  }
  const int total = 2 * nk;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (u < total)
      issue_slot((u & 1) ? xsrc : wsrc, static_cast<size_t>(u >> 1) * kRowBytes, mydst + u * kSlotBytes);
  wait_slots(min(4, total) - 2);
  barrier();
  Frags fa, fb;
  int sw = 0;
  read_frags(fa, smem, smem + kSlotBytes, aoff[0], boff[0]);
  // The first step of the tile (in whichever stage comes first: nk >= 3, 2
  // or 1) starts the accumulators from 0.
  int t = 0;
  if (nk >= 3) {
    stage<true, true, 1, true>(fa, fb, acc, sw, t, smem, mydst, wsrc, xsrc, aoff, boff);
    for (t = 1; t + 3 <= nk; ++t) stage<true, true, 1>(fa, fb, acc, sw, t, smem, mydst, wsrc, xsrc, aoff, boff);
  }
  if (t + 2 == nk) {
    if (t == 0)
      stage<false, false, 0, true>(fa, fb, acc, sw, t, smem, mydst, wsrc, xsrc, aoff, boff);
    else
      stage<false, false, 0>(fa, fb, acc, sw, t, smem, mydst, wsrc, xsrc, aoff, boff);
    ++t;
  }
  const char* ws = smem + sw * kSlotBytes;
  const char* xs = smem + ring(sw + 1) * kSlotBytes;
  if (nk == 1)
    mma_step<true, false, true>(fa, acc, fb, ws, xs, aoff[1], boff[1], wsrc, 0, mydst);
  else
    mma_step<true, false>(fa, acc, fb, ws, xs, aoff[1], boff[1], wsrc, 0, mydst);
  mma_step<false, false>(fb, acc, fa, ws, xs, 0, 0, wsrc, 0, mydst);
  // The compiler does not see the MFMAs in the assembly statements: give the
  // last ones the wait states an MFMA result needs before other instructions
  // read its registers (nothing may be scheduled across the nops).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The staging tile: row r (0..255) of 512 bytes, 16-byte chunk c stored at
// chunk position c ^ (r & 31).
__device__ __forceinline__ int stage_off(int row, int chunk) {
  return row * kStageRowBytes + ((chunk ^ (row & 31)) << 4);
}

template <bool WIDE>
__global__ void __launch_bounds__(kThreads) map_gemm_kernel(const MapParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  const int t = xcd_remap_chunked(blockIdx.x, gridDim.x);
  const TileCoord c = tile_coord<4>(t, p.tiles_m, p.tiles_n);
  const int m0 = c.tm * kTileM, n0 = c.tn * kTileN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  OpSrc<WIDE> wsrc, xsrc;
  {
    wsrc.init(p.a[c.g], static_cast<size_t>(p.N) * p.K * 2);
    xsrc.init(p.x, static_cast<size_t>(p.n_rows) * p.ld_x * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int lr = wave * 64 + j * 8 + (lane >> 3);
      const int chunk = load_chunk(lane, j);
      wsrc.set(j, (static_cast<size_t>(n0 + lr) * p.K + chunk * 8) * 2);
      int m = min(m0 + lr, p.M - 1);
      int row = p.rows[m];
      row = (row >= 0 && row < p.n_rows) ? row : 0;  // out-of-range rows read row 0, never stored
      xsrc.set(j, (static_cast<size_t>(row) * p.ld_x + chunk * 8) * 2);
    }
  }

  // This lane's bias values (4 consecutive features of each 16-feature block),
  // fetched before the main loop so their latency hides behind it.
  const int wn = wave & 1, wm = wave >> 1, r15 = lane & 15, q = lane >> 4;
  uint2 braw[8];
  {
    const uint16_t* bias = p.b[c.g] + n0 + wn * 128 + q * 4;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) braw[nb] = *reinterpret_cast<const uint2*>(bias + nb * 16);
  }

  f32x4 acc[8][8];
  mainloop(wsrc, xsrc, p.K / kBK, smem, acc);

  // Epilogue: + b, round to bf16, stage, 16-byte row stores into Y_g.  A lane
  // holds 4 consecutive features (8 bytes, one half of a staged chunk) of a row.
  // With p.ssq the squares of the stored bf16 values are summed per row as
  // well (for the norm of the next contraction): per lane over its 32
  // features, then over the four lanes of the row, then the two waves of the
  // tile's feature halves meet in LDS.
  __syncthreads();  // every wave is done reading the operand stages
  float sq[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) sq[mb] = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const float b0 = bf16_to_f32(braw[nb].x & 0xffff), b1 = bf16_to_f32(braw[nb].x >> 16);
    const float b2 = bf16_to_f32(braw[nb].y & 0xffff), b3 = bf16_to_f32(braw[nb].y >> 16);
    const int chunk = wn * 16 + nb * 2 + (q >> 1);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int row = wm * 128 + mb * 16 + r15;
      const f32x4& v = acc[nb][mb];
      uint2 o;
      o.x = pack_bf16x2(v[0] + b0, v[1] + b1);
      o.y = pack_bf16x2(v[2] + b2, v[3] + b3);
      *reinterpret_cast<uint2*>(smem + stage_off(row, chunk) + (q & 1) * 8) = o;
      sq[mb] = sq4(sq[mb], o.x, o.y);
    }
  }
  float* const sq_lds = reinterpret_cast<float*>(smem + kSlotOffset);  // [2][256], past the staging tile
  if (p.ssq) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      float t = sq[mb] + __shfl_xor(sq[mb], 16);
      t += __shfl_xor(t, 32);
      if (q == 0) sq_lds[wn * 256 + wm * 128 + mb * 16 + r15] = t;
    }
  }
  __syncthreads();
  if (p.ssq && m0 + static_cast<int>(threadIdx.x) < p.M)
    p.ssq[(static_cast<size_t>(c.g) * p.tiles_n + c.tn) * p.M + m0 + threadIdx.x] =
        sq_lds[threadIdx.x] + sq_lds[256 + threadIdx.x];
  uint16_t* y = p.y + static_cast<size_t>(c.g) * p.M * p.N;
  const int chunk = threadIdx.x & 31;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int row = it * 8 + (threadIdx.x >> 5);
    const int m = m0 + row;
    if (m < p.M) {
      const uint4 v = *reinterpret_cast<const uint4*>(smem + stage_off(row, chunk));
      store16_nt(y + static_cast<size_t>(m) * p.N + n0 + chunk * 8, v);
    }
  }
}

// Norm factor per row from the map contraction's per-tile sums of squares,
// summed in tile order (deterministic).
__global__ void __launch_bounds__(256) row_scale_kernel(const float* __restrict__ ssq, int tiles, int M,
                                                        float inv_k, float eps, float* __restrict__ rs) {
  const int g = blockIdx.y;
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const float* src = ssq + static_cast<size_t>(g) * tiles * M + m;
  float t = 0.0f;
  for (int j = 0; j < tiles; ++j) t += src[static_cast<size_t>(j) * M];
  rs[static_cast<size_t>(g) * M + m] = rsqrtf(t * inv_k + eps);
}

// Norm factor of rows that do not come from the map contraction: one wave per
// row, with the sums formed exactly as the map epilogue and row_scale_kernel
// form them (see sq4): lane l takes part q = l & 3 of half (l >> 2) & 1 of
// tile 8 i + (l >> 3) in round i.
__global__ void __launch_bounds__(256) row_rms_kernel(const RmsParams p) {
  const int g = blockIdx.y;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= p.M) return;  // whole waves leave together
  int row = p.in_rows ? p.in_rows[m] : m;
  row = (row >= 0 && row < p.n_in_rows) ? row : 0;
  const uint16_t* src = p.in[g] + static_cast<size_t>(row) * p.ld_in;
  const int tiles = p.K / kTileN;
  const int q = lane & 3, half = (lane >> 2) & 1, jj = lane >> 3;
  float total = 0.0f;
  for (int i = 0; i * 8 < tiles; ++i) {
    const int j = min(i * 8 + jj, tiles - 1);  // lanes past the last tile load it again, unused
    const uint16_t* t0 = src + j * kTileN + half * 128 + q * 4;
    float s_ = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint2 v = *reinterpret_cast<const uint2*>(t0 + nb * 16);
      s_ = sq4(s_, v.x, v.y);
    }
    float t = s_ + __shfl_xor(s_, 1);
    t += __shfl_xor(t, 2);
    t += __shfl_xor(t, 4);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float v = __shfl(t, k * 8);
      if (i * 8 + k < tiles) total += v;
    }
  }
  if (lane == 0) p.rs[static_cast<size_t>(g) * p.M + m] = rsqrtf(total * p.inv_k + p.eps);
}

// ---- Indexer-key remainder: a "tall" tile of 128 features x 512 rows --------
// When the indexer key columns end half way into a 256-feature tile (one
// 128-wide head, or an odd count of them), that tile would be half zero
// padding.  A tall tile of kv_gemm_kernel's launch computes those 128
// features alone, for the 512 rows of two row tiles: each of the 4 waves owns
// 128 features x 128 rows (the same 8x8 blocks of v_mfma_f32_16x16x32_bf16 and lane layout as the
// main loop), all waves share the weight fragments.  LDS holds two buffers of
// one 64-column stage each: 128 weight rows (16 KB) then 512 data rows
// (64 KB), rows of 128 bytes with the main loop's chunk swizzle.  Each wave
// loads and reads only its own 128 data rows, so it loads stage t+2's rows
// into stage t's buffer as soon as its own reads of them have returned, half
// way through stage t's first step; the weight rows, which every wave reads,
// follow in the second step, after the barrier that ends all reads of stage t.
constexpr int kTallRows = 512;
constexpr int kTallA = 128 * kRowBytes;               // 16 KB of weight rows
constexpr int kTallBuf = kTallA + kTallRows * kRowBytes;  // 80 KB per stage buffer
constexpr int kTallLoads = 20;                        // per wave per stage: 4 weight + 16 data
constexpr int kTallStageRow = 128 * 2;                // 256 B per staged output row
constexpr int kTallSlotOffset = kTallRows * kTallStageRow;  // 128 KB, then 512 int32 slot ids
static_assert(2 * kTallBuf <= kLdsBytes && kTallSlotOffset + kTallRows * 4 <= 2 * kTallBuf, "tall tile LDS");

__device__ __forceinline__ void tall_wait(int loads) {
  if (loads == 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (loads == 16)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
}
static_assert(kTallLoads == 20, "tall_wait immediates assume 20 loads per stage");

// Where the 20 loads of a stage read: a raw buffer resource per operand (the
// layer's prepared weights, its input rows) plus a 32-bit byte offset per
// lane and load, so the loads take one VGPR of address each (the host uses
// tall tiles only when every layer input spans less than 4 GiB).
struct TallSrc {
  __amdgpu_buffer_rsrc_t w, x;
  uint32_t off[kTallLoads];
};

// The 20 loads of one stage for this wave into buffer `buf`: j < 4 weight rows
// 32 w + 8 j + i / 8, j >= 4 data rows 128 w + 8 (j - 4) + i / 8 (lane i lands
// at position i % 8 of its row).
__device__ __forceinline__ void tall_load(int j, const TallSrc& src, size_t kbyte, char* buf, int wave) {
  char* dst = j < 4 ? buf + (32 * wave + 8 * j) * kRowBytes
                    : buf + kTallA + (128 * wave + 8 * (j - 4)) * kRowBytes;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 4 ? src.w : src.x, (lds_ptr_t*)dst, 16, src.off[j],
                                           static_cast<int>(kbyte), 0, 0);
}

// One 32-column step on fragments f from buffer `cur`; READ: the 16 fragment
// reads of the next step (from `nbuf` at offsets aoff / boff) follow MFMAs
// 0..15; LOAD: the 20 loads of a stage (into `lbuf`) follow MFMAs 4, 7, ..., 61.
// LOADX (step 0): once this wave's own fragment reads have returned (after
// MFMA 23), the 16 loads of its quarter of the data rows follow MFMAs 24, 26,
// ..., 54 (no other wave reads or writes that quarter, so no barrier is
// needed); LOADA (step 1, after the barrier): the 4 weight-row loads follow
// MFMAs 16, 28, 40, 52.
template <bool READ, bool LOADX, bool LOADA, bool FIRST>
__device__ __forceinline__ void tall_step(const Frags& f, f32x4 (&acc)[8][8], Frags& nf, const char* nbuf, int aoff,
                                          int boff, const TallSrc& src, size_t kbyte, char* lbuf, int wave) {
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const int nb = i >> 3, mb = mfma_col(i);
    if (FIRST)
      mfma16_first(acc[nb][mb], f.a[nb], f.b[mb]);
    else
      mfma16(acc[nb][mb], f.a[nb], f.b[mb]);
    if (READ && i < 8) nf.a[i] = *reinterpret_cast<const bf16x8*>(nbuf + aoff + i * 16 * kRowBytes);
    if (READ && i >= 8 && i < 16)
      nf.b[i - 8] = *reinterpret_cast<const bf16x8*>(nbuf + kTallA + boff + (i - 8) * 16 * kRowBytes);
    if (LOADX && i == 23) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (LOADX && i >= 24 && (i - 24) % 2 == 0 && i <= 54) tall_load(4 + (i - 24) / 2, src, kbyte, lbuf, wave);
    if (LOADA && i >= 16 && (i - 16) % 12 == 0 && i <= 52) tall_load((i - 16) / 12, src, kbyte, lbuf, wave);
  }
}

// Stage t from buffer t % 2: step 0 reads step 1's fragments from the same
// buffer; the wave's loads of stage t+1 have landed (vmcnt) and the barrier
// publishes them and ends every read of buffer t % 2; step 1 reads stage
// t+1's first fragments and loads stage t+2 into buffer t % 2.
template <bool NEXT, bool LOAD, bool FIRST>
__device__ __forceinline__ void tall_stage(Frags& fa, Frags& fb, f32x4 (&acc)[8][8], int t, char* smem,
                                           const TallSrc& src, const int (&aoff)[2], const int (&boff)[2], int wave) {
  char* cur = smem + (t & 1) * kTallBuf;
  char* nxt = smem + ((t + 1) & 1) * kTallBuf;
  const size_t kb = static_cast<size_t>(t + 2) * kRowBytes;
  tall_step<true, LOAD, false, FIRST>(fa, acc, fb, cur, aoff[1], boff[1], src, kb, cur, wave);
  if (NEXT) {
    tall_wait(LOAD ? 16 : 0);  // stage t+1 landed; this stage's data-row loads may fly
    barrier();
  }
  tall_step<NEXT, false, LOAD, false>(fb, acc, fa, nxt, aoff[0], boff[0], src, kb, cur, wave);
}

// One tall tile: layer g, rows m0 .. m0 + 511 of the call, features
// [tall_f0, tall_f0 + 128) of the prepared weights; smem is the workgroup's LDS.
template <int HD>
__device__ __forceinline__ void tall_tile(const KvParams& p, int g, int m0, char* smem) {
  int* const slot_of = reinterpret_cast<int*>(smem + kTallSlotOffset);
  const int f0 = p.tall_f0;  // first prepared-weight row (feature) of the tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r15 = lane & 15, q = lane >> 4;

  TallSrc src;
  src.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.wkv + static_cast<size_t>(g) * p.wrows * p.K),
                                            static_cast<short>(0), static_cast<int>(static_cast<uint32_t>(
                                                static_cast<size_t>(p.wrows) * p.K * 2)), 0x00020000);
  src.x = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.in[g]), static_cast<short>(0),
                                            static_cast<int>(static_cast<uint32_t>(
                                                static_cast<size_t>(p.n_in_rows) * p.ld_in * 2)), 0x00020000);
#pragma unroll
  for (int j = 0; j < kTallLoads; ++j) {
    const int chunk = load_chunk(lane, j);
    if (j < 4) {
      const int lr = 32 * wave + 8 * j + (lane >> 3);
      src.off[j] = static_cast<uint32_t>((static_cast<size_t>(f0 + lr) * p.K + chunk * 8) * 2);
    } else {
      const int lr = 128 * wave + 8 * (j - 4) + (lane >> 3);
      const int m = min(m0 + lr, p.M - 1);
      int row = p.in_rows ? p.in_rows[m] : m;
      row = (row >= 0 && row < p.n_in_rows) ? row : 0;
      src.off[j] = static_cast<uint32_t>((static_cast<size_t>(row) * p.ld_in + chunk * 8) * 2);
    }
  }

  // fragment offsets: weight rows 16 nb + r15 (shared), data rows 128 w + 16 mb + r15
  int aoff[2], boff[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    aoff[st] = slot_pos(r15, 4 * st + q);
    boff[st] = slot_pos(wave * 128 + r15, 4 * st + q);
  }
  f32x4 acc[8][8];
  const int nk = p.K / kBK;
#pragma unroll
  for (int j = 0; j < kTallLoads; ++j) tall_load(j, src, 0, smem, wave);
  if (nk > 1) {
#pragma unroll
    for (int j = 0; j < kTallLoads; ++j) tall_load(j, src, kRowBytes, smem + kTallBuf, wave);
    tall_wait(20);
  } else {
    tall_wait(0);
  }
  barrier();
  Frags fa, fb;
#pragma unroll
  for (int i = 0; i < 8; ++i) fa.a[i] = *reinterpret_cast<const bf16x8*>(smem + aoff[0] + i * 16 * kRowBytes);
#pragma unroll
  for (int i = 0; i < 8; ++i) fa.b[i] = *reinterpret_cast<const bf16x8*>(smem + kTallA + boff[0] + i * 16 * kRowBytes);
  // stage 0 starts the accumulators from 0; stages t <= nk-3 load stage t+2
  if (nk >= 3) {
    tall_stage<true, true, true>(fa, fb, acc, 0, smem, src, aoff, boff, wave);
    for (int t = 1; t + 3 <= nk; ++t) tall_stage<true, true, false>(fa, fb, acc, t, smem, src, aoff, boff, wave);
    tall_stage<true, false, false>(fa, fb, acc, nk - 2, smem, src, aoff, boff, wave);
    tall_stage<false, false, false>(fa, fb, acc, nk - 1, smem, src, aoff, boff, wave);
  } else if (nk == 2) {
    tall_stage<true, false, true>(fa, fb, acc, 0, smem, src, aoff, boff, wave);
    tall_stage<false, false, false>(fa, fb, acc, 1, smem, src, aoff, boff, wave);
  } else {
    tall_stage<false, false, true>(fa, fb, acc, 0, smem, src, aoff, boff, wave);
  }
  // the accumulators are read only after the wait states an MFMA result needs
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // row bookkeeping as in kv_gemm_kernel: bad rows get slot -1 and are not stored
  int orow[8], pos[8], slot_r[8];
  float rs[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int m = min(m0 + wave * 128 + mb * 16 + r15, p.M - 1);
    orow[mb] = p.out_rows ? p.out_rows[m] : m;
    rs[mb] = p.rs[g][m];
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int r = orow[mb];
    const bool ok = (m0 + wave * 128 + mb * 16 + r15 < p.M) & (r >= 0) & (r < p.n_rows);
    orow[mb] = ok ? r : 0;
    slot_r[mb] = ok ? 0 : -1;
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) pos[mb] = p.positions[orow[mb]];
  if (p.slots) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) slot_r[mb] = slot_r[mb] < 0 ? -1 : p.slots[orow[mb]];
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) slot_r[mb] = slot_r[mb] < 0 ? -1 : orow[mb];
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const bool good = (slot_r[mb] >= 0) & (pos[mb] >= 0) & (pos[mb] < p.max_pos) & (slot_r[mb] < p.n_slots);
    slot_r[mb] = good ? slot_r[mb] : -1;
    pos[mb] = good ? pos[mb] : 0;
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // every wave is done with the operand buffers
  if (q == 0) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) slot_of[wave * 128 + mb * 16 + r15] = slot_r[mb];
  }
  // RoPE over the 128 features (one head of 128 or two of 64), scaled by the
  // row's norm factor, rounded, staged: row r of 256 bytes, 16-byte chunk c
  // at position c ^ (r & 15).
  constexpr int half = HD / 2;
  constexpr int pstep = half / 16;
  const float2* tab = reinterpret_cast<const float2*>(p.rope);
  auto stage4 = [&](int nb, int mb, float v0, float v1, float v2, float v3) {
    const int row = wave * 128 + mb * 16 + r15;
    const int chunk = nb * 2 + (q >> 1);
    uint2 o;
    o.x = pack_bf16x2(v0, v1);
    o.y = pack_bf16x2(v2, v3);
    *reinterpret_cast<uint2*>(smem + row * kTallStageRow + ((chunk ^ (row & 15)) << 4) + (q & 1) * 8) = o;
  };
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int jb = (nb * 16) & (HD - 1);
    if (jb >= half) continue;
    const int nb2 = nb + pstep;
    float4 cs[8][2];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const float2* trow = tab + static_cast<size_t>(pos[mb]) * half + jb + q * 4;
      cs[mb][0] = *reinterpret_cast<const float4*>(trow);
      cs[mb][1] = *reinterpret_cast<const float4*>(trow + 2);
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const float c4[8] = {cs[mb][0].x, cs[mb][0].y, cs[mb][0].z, cs[mb][0].w,
                           cs[mb][1].x, cs[mb][1].y, cs[mb][1].z, cs[mb][1].w};
      float y1[4], y2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x1 = agpr(acc[nb][mb][i]) * rs[mb];
        const float x2 = agpr(acc[nb2][mb][i]) * rs[mb];
        rotate(x1, x2, c4[2 * i], c4[2 * i + 1], y1[i], y2[i]);
      }
      stage4(nb, mb, y1[0], y1[1], y1[2], y1[3]);
      stage4(nb2, mb, y2[0], y2[1], y2[2], y2[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  const int chunk = threadIdx.x & 15;
  uint16_t* dst_base = p.ic[g] + (f0 - 2 * p.w) + chunk * 8;
#pragma unroll 4
  for (int it = 0; it < kTallRows / 16; ++it) {
    const int row = it * 16 + (threadIdx.x >> 4);
    const int slot = slot_of[row];
    if (slot >= 0) {
      const uint4 v = *reinterpret_cast<const uint4*>(smem + row * kTallStageRow + ((chunk ^ (row & 15)) << 4));
      store16_nt(dst_base + static_cast<size_t>(slot) * p.widx, v);
    }
  }
}

// VSCALE: the value rescale is applied; QK: keys are RMS-normalised per head
// with a per-dimension gain before RoPE.  Each option is its own
// instantiation, so the plain fill's epilogue keeps its register budget.
template <int HD, bool VSCALE, bool QK, bool WIDE>
__global__ void __launch_bounds__(kThreads) kv_gemm_kernel(const KvParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  int* const slot_of = reinterpret_cast<int*>(smem + kSlotOffset);
  const int t = xcd_remap_contiguous(blockIdx.x, gridDim.x);
  TileCoord c;
  if (p.tall_f0 >= 0) {
    // Each group of (up to) two row tiles is one tall tile of the indexer
    // remainder, then its tiles_n regular tiles; the tall tile's rows are the
    // ones the group's regular tiles read at the same time, so its loads of
    // them mostly hit L2.
    const int full = p.tiles_m / 2;
    const int per_group = 2 * p.tiles_n + 1;
    const int per_layer = p.tiles_m * p.tiles_n + (p.tiles_m + 1) / 2;
    const int g = t / per_layer;
    const int u = t - g * per_layer;
    const int grp = u < full * per_group ? u / per_group : full;
    const int v = u - grp * per_group;
    const int gsz = min(p.tiles_m - 2 * grp, 2);
    if (v == 0) {
      tall_tile<HD>(p, g, grp * 2 * kTileM, smem);
      return;
    }
    c.g = g;
    c.tm = 2 * grp + (v - 1) % gsz;
    c.tn = (v - 1) / gsz;
  } else {
    c = tile_coord_rt(t, p.tiles_m, p.tiles_n, p.group_m);
  }
  const int m0 = c.tm * kTileM, n0 = c.tn * kTileN + (p.v_only ? p.w / kTileN * kTileN : 0);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  OpSrc<WIDE> wsrc, xsrc;
  {
    wsrc.init(p.wkv + static_cast<size_t>(c.g) * p.wrows * p.K, static_cast<size_t>(p.wrows) * p.K * 2);
    xsrc.init(p.in[c.g], static_cast<size_t>(p.n_in_rows) * p.ld_in * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int lr = wave * 64 + j * 8 + (lane >> 3);
      const int chunk = load_chunk(lane, j);
      wsrc.set(j, (static_cast<size_t>(n0 + lr) * p.K + chunk * 8) * 2);
      const int m = min(m0 + lr, p.M - 1);
      int row = p.in_rows ? p.in_rows[m] : m;
      row = (row >= 0 && row < p.n_in_rows) ? row : 0;
      xsrc.set(j, (static_cast<size_t>(row) * p.ld_in + chunk * 8) * 2);
    }
  }

  const int wn = wave & 1, wm = wave >> 1, r15 = lane & 15, q = lane >> 4;
  // Output-row indices and norm factors of this lane's 8 rows, fetched before
  // the main loop so their latency hides behind it (indices clamped: every
  // load is in bounds).
  int orow[8];
  float rs[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int m = min(m0 + wm * 128 + mb * 16 + r15, p.M - 1);
    orow[mb] = p.out_rows ? p.out_rows[m] : m;
    rs[mb] = p.rs[c.g][m];
  }

  f32x4 acc[8][8];
  mainloop(wsrc, xsrc, p.K / kBK, smem, acc);

  // Row bookkeeping, branch-free so that all loads of a kind issue together:
  // position, cache slot and (rescale) request of each row; a row that is out
  // of range anywhere gets slot -1 and is not stored.
  int pos[8], slot_r[8], grp_r[8];
  bool ok[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int r = orow[mb];
    ok[mb] = (m0 + wm * 128 + mb * 16 + r15 < p.M) & (r >= 0) & (r < p.n_rows);
    orow[mb] = ok[mb] ? r : 0;
  }
  // (one wave-uniform branch per array, outside the row loops, so that each
  // array's 8 loads issue back to back)
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) pos[mb] = p.positions[orow[mb]];
  if (p.slots) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) slot_r[mb] = p.slots[orow[mb]];
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) slot_r[mb] = orow[mb];
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) grp_r[mb] = VSCALE ? p.group_of_row[orow[mb]] : 0;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const bool good = ok[mb] & (pos[mb] >= 0) & (pos[mb] < p.max_pos) & (slot_r[mb] >= 0) &
                      (slot_r[mb] < p.n_slots) & (!VSCALE | ((grp_r[mb] >= 0) & (grp_r[mb] < p.n_groups)));
    slot_r[mb] = good ? slot_r[mb] : -1;
    pos[mb] = good ? pos[mb] : 0;
    grp_r[mb] = good ? grp_r[mb] : 0;
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // every wave is done with the operand slots
  if (wn == 0 && q == 0) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) slot_of[wm * 128 + mb * 16 + r15] = slot_r[mb];
  }
  // First feature of this wave; a whole wave is one kind: attention keys
  // [0, w), values [w, 2w), indexer keys [2w, 2w + widx) (rotated like keys,
  // never QK-normed), or padding past them (not stored).  With v_only a tile
  // may start inside the keys when w is not a multiple of 256; those key
  // waves are neither rotated nor stored.
  const int fw = n0 + wn * 128;
  const bool is_attn_key = fw < p.w && !p.v_only;
  const bool is_key = is_attn_key || (fw >= 2 * p.w && fw < 2 * p.w + p.widx);
  const bool is_value = fw >= p.w && fw < 2 * p.w;
  const bool qk_wave = QK && is_attn_key;
  // Value waves of a rescaled fill: the request's value scale for the wave's
  // first head (and, for heads of 64, the second head, blocks 4-7) is folded
  // into the norm's per-row factor; without a rescale the factor is exactly
  // the norm's scale.
  const float* const vsw = (VSCALE && is_value) ? p.vscale[c.g] + (fw - p.w) / HD : nullptr;
  float rs2[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) rs2[mb] = rs[mb];
  if (VSCALE && vsw) {  // wave-uniform; the 8 (16) scale loads issue together
    float sa[8], sb[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const float* sg = vsw + grp_r[mb] * p.n_kv;
      sa[mb] = sg[0];
      sb[mb] = HD == 64 ? sg[1] : 1.0f;
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      rs2[mb] = rs[mb] * sb[mb];
      rs[mb] = rs[mb] * sa[mb];
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  // Scale (and for keys rotate), round to bf16 and write each 4-feature run
  // straight into the staging tile: 8 bytes, one half of a staged chunk.
  auto stage4 = [&](int nb, int mb, float v0, float v1, float v2, float v3) {
    const int row = wm * 128 + mb * 16 + r15;
    uint2 o;
    o.x = pack_bf16x2(v0, v1);
    o.y = pack_bf16x2(v2, v3);
    *reinterpret_cast<uint2*>(smem + stage_off(row, wn * 16 + nb * 2 + (q >> 1)) + (q & 1) * 8) = o;
  };
  if (is_key) {
    // RoPE, rotate-half: feature j < hd/2 of a head pairs with j + hd/2.  A
    // wave spans 128 features = one head of 128 or two heads of 64, so the
    // partner is block nb + hd/32 at the same register index.
    constexpr int half = HD / 2;
    constexpr int pstep = half / 16;  // 4 for hd 128, 2 for hd 64
    constexpr int heads = 128 / HD;   // heads per wave
    constexpr int per_head = HD / 16; // 16-feature blocks per head
    const float2* tab = reinterpret_cast<const float2*>(p.rope);
    // With QK-norm each head is also divided by sqrt(mean over the head of
    // k^2 + eps) and its dimensions scaled by the gain before the rotation.
    // The head sums come first (a lane holds a quarter of each head's values
    // for its row, the rest are in lanes ^ 16, ^ 32, ^ 48); the division
    // then folds into the row factor of the rotation pass.
    float kf[8][heads];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int h = 0; h < heads; ++h) kf[mb][h] = rs[mb];
    if (qk_wave) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int h = 0; h < heads; ++h) {
          float sq = 0.0f;
#pragma unroll
          for (int nb = h * per_head; nb < (h + 1) * per_head; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = agpr(acc[nb][mb][i]) * rs[mb];
              sq += x * x;
            }
          sq += __shfl_xor(sq, 16);
          sq += __shfl_xor(sq, 32);
          kf[mb][h] = rs[mb] * rsqrtf(sq * (1.0f / HD) + p.eps);
        }
      }
    }
    const uint16_t* kg = QK ? p.kgamma[c.g] : nullptr;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int jb = (nb * 16) & (HD - 1);
      if (jb >= half) continue;
      const int nb2 = nb + pstep;
      const int h = nb / per_head;
      // cos/sin of dims jb + 4q .. + 3 for the 8 rows, all requested at once
      float4 cs[8][2];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const float2* trow = tab + static_cast<size_t>(pos[mb]) * half + jb + q * 4;
        cs[mb][0] = *reinterpret_cast<const float4*>(trow);
        cs[mb][1] = *reinterpret_cast<const float4*>(trow + 2);
      }
      float g1[4] = {1.0f, 1.0f, 1.0f, 1.0f}, g2[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if (qk_wave) {
        // gains of dimensions j and j + hd/2, four consecutive each
        const uint2 a = *reinterpret_cast<const uint2*>(kg + jb + q * 4);
        const uint2 b = *reinterpret_cast<const uint2*>(kg + jb + half + q * 4);
        g1[0] = __uint_as_float(a.x << 16), g1[1] = __uint_as_float(a.x & 0xffff0000u);
        g1[2] = __uint_as_float(a.y << 16), g1[3] = __uint_as_float(a.y & 0xffff0000u);
        g2[0] = __uint_as_float(b.x << 16), g2[1] = __uint_as_float(b.x & 0xffff0000u);
        g2[2] = __uint_as_float(b.y << 16), g2[3] = __uint_as_float(b.y & 0xffff0000u);
      }
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const float c4[8] = {cs[mb][0].x, cs[mb][0].y, cs[mb][0].z, cs[mb][0].w,
                             cs[mb][1].x, cs[mb][1].y, cs[mb][1].z, cs[mb][1].w};
        float y1[4], y2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x1 = agpr(acc[nb][mb][i]) * kf[mb][h] * g1[i];
          const float x2 = agpr(acc[nb2][mb][i]) * kf[mb][h] * g2[i];
          rotate(x1, x2, c4[2 * i], c4[2 * i + 1], y1[i], y2[i]);
        }
        stage4(nb, mb, y1[0], y1[1], y1[2], y1[3]);
        stage4(nb2, mb, y2[0], y2[1], y2[2], y2[3]);
      }
      // keep the accumulator reads of later blocks from being hoisted here
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const float f = (HD == 64 && nb >= 4) ? rs2[mb] : rs[mb];
        stage4(nb, mb, agpr(acc[nb][mb][0]) * f, agpr(acc[nb][mb][1]) * f, agpr(acc[nb][mb][2]) * f,
               agpr(acc[nb][mb][3]) * f);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  const int chunk = threadIdx.x & 31;
  const int f = n0 + chunk * 8;
  const bool store = !(p.v_only && f < p.w) && f < 2 * p.w + p.widx;
  uint16_t* dst_base = f < p.w       ? p.kc[c.g] + f
                       : f < 2 * p.w ? p.vc[c.g] + (f - p.w)
                                     : p.ic[c.g] + (f - 2 * p.w);
  const int stride = f < 2 * p.w ? p.w : p.widx;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int row = it * 8 + (threadIdx.x >> 5);
    const int slot = slot_of[row];
    if (slot >= 0 && store) {
      const uint4 v = *reinterpret_cast<const uint4*>(smem + stage_off(row, chunk));
      store16_nt(dst_base + static_cast<size_t>(slot) * stride, v);
    }
  }
}

// Prepared weights: one thread per 8 consecutive inputs of one output feature.
__global__ void __launch_bounds__(256) prep_kv_kernel(const PrepParams p) {
  const int g = blockIdx.y;
  const int per_row = p.d >> 3;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(p.rows) * per_row) return;
  const int f = static_cast<int>(idx / per_row);
  const int k8 = static_cast<int>(idx - static_cast<int64_t>(f) * per_row) * 8;
  uint16_t* dst = p.out + (static_cast<size_t>(g) * p.rows + f) * p.d + k8;
  if (f >= 2 * p.w + p.widx) {  // padding rows of the last tile
    *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint16_t* src = f < p.w       ? p.wk[g] + static_cast<size_t>(f) * p.d
                        : f < 2 * p.w ? p.wv[g] + static_cast<size_t>(f - p.w) * p.d
                                      : p.wi[g] + static_cast<size_t>(f - 2 * p.w) * p.d;
  const uint4 wr = *reinterpret_cast<const uint4*>(src + k8);
  const uint4 gr = *reinterpret_cast<const uint4*>(p.gamma[g] + k8);
  const uint32_t wv[4] = {wr.x, wr.y, wr.z, wr.w};
  const uint32_t gv[4] = {gr.x, gr.y, gr.z, gr.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_to_f32(wv[i] & 0xffff) * bf16_to_f32(gv[i] & 0xffff);
    const float hi = bf16_to_f32(wv[i] >> 16) * bf16_to_f32(gv[i] >> 16);
    o[i] = pack_bf16x2(lo, hi);
  }
  *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
}

// (cos, sin) of pos * theta^(-2j/hd), formed and evaluated in double precision.
__global__ void __launch_bounds__(256) rope_table_kernel(float2* tab, int max_pos, int hd, double theta) {
  const int half = hd >> 1;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(max_pos) * half) return;
  const int p = static_cast<int>(idx / half);
  const int j = static_cast<int>(idx - static_cast<int64_t>(p) * half);
  const double freq = pow(theta, -2.0 * j / hd);
  const double ang = static_cast<double>(p) * freq;
  tab[idx] = make_float2(static_cast<float>(cos(ang)), static_cast<float>(sin(ang)));
}

__global__ void __launch_bounds__(256) clear_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void __launch_bounds__(256) validate_kernel(const int32_t* rows, int n, int n_rows, int ascending,
                                                       const int32_t* positions, int max_pos,
                                                       const int32_t* slots, int n_slots, int32_t* flag) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = rows[i];
  int bits = 0;
  if (r < 0 || r >= n_rows) {
    bits |= 1;
  } else {
    const int ps = positions[r];
    if (ps < 0 || ps >= max_pos) bits |= 2;
    const int s = slots ? slots[r] : r;
    if (s < 0 || s >= n_slots) bits |= 4;
  }
  if (ascending && i > 0 && rows[i - 1] >= r) bits |= 8;
  if (bits) atomicOr(flag, bits);
}

}  // namespace

// An operand read through a buffer resource must lie within 4 GiB of its base.
static bool spans_4g(int64_t rows, int64_t ld) { return rows * ld * 2 >= (int64_t(1) << 32); }

hipError_t launch_map(const MapParams& p, int n_layers, hipStream_t s) {
  const int grid = n_layers * p.tiles_m * p.tiles_n;
  if (spans_4g(p.N, p.K) || spans_4g(p.n_rows, p.ld_x))
    hipLaunchKernelGGL(map_gemm_kernel<true>, dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(map_gemm_kernel<false>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_row_scale(const float* ssq, int tiles, int M, int n_layers, float inv_k, float eps, float* rs,
                            hipStream_t s) {
  if (M <= 0 || n_layers <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_scale_kernel, dim3((M + 255) / 256, n_layers), dim3(256), 0, s, ssq, tiles, M, inv_k, eps, rs);
  return hipGetLastError();
}

hipError_t launch_row_rms(const RmsParams& p, int n_layers, hipStream_t s) {
  if (p.M <= 0 || n_layers <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_rms_kernel, dim3((p.M + 3) / 4, n_layers), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool WIDE>
static void launch_kv_variant(const KvParams& p, int grid, hipStream_t s) {
  const int variant = (p.head_dim == 128 ? 4 : 0) | (p.group_of_row ? 2 : 0) | (p.qk_norm ? 1 : 0);
  switch (variant) {
    case 0: hipLaunchKernelGGL((kv_gemm_kernel<64, false, false, WIDE>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 1: hipLaunchKernelGGL((kv_gemm_kernel<64, false, true, WIDE>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((kv_gemm_kernel<64, true, false, WIDE>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 3: hipLaunchKernelGGL((kv_gemm_kernel<64, true, true, WIDE>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL((kv_gemm_kernel<128, false, false, WIDE>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 5: hipLaunchKernelGGL((kv_gemm_kernel<128, false, true, WIDE>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case 6: hipLaunchKernelGGL((kv_gemm_kernel<128, true, false, WIDE>), dim3(grid), dim3(kThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((kv_gemm_kernel<128, true, true, WIDE>), dim3(grid), dim3(kThreads), 0, s, p); break;
  }
}

hipError_t launch_kv(const KvParams& p_in, int n_layers, hipStream_t s) {
  KvParams p = p_in;
  p.group_m = (p.tiles_n * 4 <= 32 && 32 % p.tiles_n == 0) ? 4 : 2;
  // tall tiles only for indexer columns past the keys and values (a value-
  // initialised KvParams has tall_f0 = 0, which means none)
  if (p.v_only || p.widx == 0 || p.tall_f0 < 2 * p.w) p.tall_f0 = -1;
  const int grid = n_layers * (p.tiles_m * p.tiles_n + (p.tall_f0 >= 0 ? (p.tiles_m + 1) / 2 : 0));
  const bool wide = spans_4g(p.wrows, p.K) || spans_4g(p.n_in_rows, p.ld_in);
  if (wide)
    launch_kv_variant<true>(p, grid, s);
  else
    launch_kv_variant<false>(p, grid, s);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepParams& p, int n_layers, hipStream_t s) {
  const int64_t per_layer = static_cast<int64_t>(p.rows) * (p.d >> 3);
  const int blocks = static_cast<int>((per_layer + 255) / 256);
  hipLaunchKernelGGL(prep_kv_kernel, dim3(blocks, n_layers), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* table, int max_pos, int head_dim, double theta, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(max_pos) * (head_dim / 2);
  const int blocks = static_cast<int>((n + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<float2*>(table),
                     max_pos, head_dim, theta);
  return hipGetLastError();
}

hipError_t launch_validate(const int32_t* rows, int n, int n_rows, int ascending, const int32_t* positions,
                           int max_pos, const int32_t* slots, int n_slots, int32_t* flag, hipStream_t s) {
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(256), 0, s, flag, 1);
  if (n > 0)
    hipLaunchKernelGGL(validate_kernel, dim3((n + 255) / 256), dim3(256), 0, s, rows, n, n_rows, ascending,
                       positions, max_pos, slots, n_slots, flag);
  return hipGetLastError();
}

}  // namespace rf
