// Mamba2 temporal scan, forward and backward, hand-written for gfx950 (MI355X).
//
// What is computed (foxhunt "Custom Kernel Optimization Implementation Plan",
// Tasks 1-2; design spec "cuBLAS Projections + Batch-Parallel Scans", Design
// section 1): the projections a = H W_A, b = H W_B, c = h_s2 W_C, the gated
// recurrence x_{t+1} = sigmoid(a_t) x_t + b_t from x_0 = 0, context = c * x_K,
// and for L = sum(d_context * context) the weight gradients
// dW_A = H^T d_a, dW_B = H^T d_b, dW_C = h_s2^T d_c.
//
// Design (the pages' cuBLAS-plus-scan split is prior art, not followed):
//
//  * fwd_kernel: one work-group per (block of 16 samples, group of 16 states).
//    W_A and W_B of the state group sit in LDS, each weight split exactly
//    into three bf16 terms, in the v_mfma_f32_16x16x32_bf16 B-operand layout.
//    Each of the 8 waves projects one history step of the 16 samples
//    (M = samples, N = states, K = trunk features), streaming every
//    h_history row from HBM once as 8 rows x 128 B per load, through a
//    per-wave LDS tile into the operand order, where each value is split
//    into three bf16 terms too; six of the nine term products accumulate in
//    fp32.  The a|b tiles meet in LDS, where 4 waves run the recurrence, one
//    lane per (sample, state), in registers.  The readout c (fp32 MFMAs, W_C
//    read from memory) is split over the waves by trunk chunk and summed in
//    a fixed order.
//
//  * The backward needs no sequential scan.  With P_t = prod_{v>t} g_v,
//      d_b_t = d_context * (c P_t),   d_a_t = d_context * (c P_t x_t g_t (1-g_t)),
//      d_c   = d_context * x_K,
//    so the forward stores beta_t = c P_t, alpha_t = beta_t x_t g_t (1-g_t)
//    and x_K ("saved"), and the backward only scales them by d_context.
//    When K spans several 8-step rounds the forward stores each round's
//    terms relative to the end of that round, plus one factor per round (the
//    product of all later gates), which the backward multiplies in; so no
//    pass over earlier rounds' terms is ever needed.
//
//  * bwd_partials_kernel: split-K tall reduction.  One work-group per
//    (64-feature column block, state group, range of sample blocks); its 12
//    waves take (sample block, history step) units round-robin and accumulate
//    H^T [d_a | d_b] and h_s2^T d_c with MFMA (M = features, N = states,
//    K = rows) in registers: fp32 MFMAs with one state group, split-bf16
//    MFMAs over pairs of steps with several (where the four state groups'
//    work-groups make the contraction bound by the matrix cores and the
//    VALU).  The waves' partials are summed in LDS in a fixed
//    order and written as one slice.  Work-groups that share rows are placed
//    on the same XCD (dispatch is round-robin over the 8 XCDs) so the shared
//    saved/d_context reads hit that XCD's L2.
//
//  * bwd_reduce_kernel: sums the slices in a fixed order, overwriting dW.
//    No floating-point atomics anywhere, so results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "mamba2_scan.h"

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

namespace {

constexpr int kGroup = 16;       // states per state group (MFMA N)
constexpr int kBlock = 16;       // samples per block (MFMA M in the forward)
constexpr int kPlane = kBlock * kGroup;  // floats in one (sample, state) plane
constexpr int kColBlock = 64;    // trunk features per backward column block
constexpr int kFwdWaves = 8;
constexpr int kChunk = kFwdWaves;  // history steps projected per forward round
// Sample blocks per forward work-group: two when the weight slab is so large
// (SH2 >= 320) that two one-block work-groups would not fit a CU's LDS, so a
// CU still runs sixteen forward waves; one otherwise (two work-groups per
// CU, which measured faster there).
__host__ __device__ constexpr int fwd_blocks(int nkc) { return nkc >= 20 ? 2 : 1; }
constexpr int kFwdPrefetch = 4;    // fp32 history loads each forward wave keeps in flight
constexpr int kCUs = 256;            // compute units of an MI355X
constexpr int kFwdPairPrefetch = 4;  // bf16 history loads (64 features of 8 rows) each wave keeps in flight
constexpr int kRegRounds = 8;      // rounds whose gate product the forward keeps in registers
constexpr int kFwdChunkTarget = 512;  // forward work-groups a chunked history aims for
constexpr int kBwdWaves = 12;
constexpr int kBwdPairWaves = 8;  // paired-step units (STATE_D >= 32): two units of registers per wave
constexpr int kBwdTargetGroups = 256;  // backward work-groups to aim for (one per CU)
constexpr int kRedThreads = 256;
constexpr int kRedQuads = 32;      // output float4s per reduce work-group
constexpr int kRedGroups = kRedThreads / kRedQuads;  // slice groups per output

__device__ __forceinline__ v4f mfma16x16x4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f ld4(const float* p) { return *reinterpret_cast<const v4f*>(p); }

// Streaming accesses: data read once per kernel (h_history, h_s2) and results
// no kernel reads back soon (context, saved terms, split-K slices) carry the
// non-temporal hint, so they do not displace the lines that are reused (the
// weight slab, the saved planes shared by the column blocks).
__device__ __forceinline__ v4f ld4_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
}
__device__ __forceinline__ void st_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }

// Trunk inputs (h_history, h_s2) come as fp32 or as bf16 bit patterns; either
// way four consecutive elements arrive as one streamed load and widen to fp32
// exactly (a bf16 value is the top half of the fp32 with the same value).
typedef unsigned short bf16_t;
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
template <class T>
__device__ __forceinline__ v4f ld4_in(const T* p);
template <>
__device__ __forceinline__ v4f ld4_in<float>(const float* p) {
  return ld4_stream(p);
}
// Eight consecutive bf16 values as one 16-byte streamed load, widened into
// two groups of four.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
// Two floats to two bf16 (round to nearest even) in one word, a's in the low half.
__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((v2f_t){a, b}, v2bf_t));
}
// Exact three-term bf16 split of two floats, packed: a = h + m + l (low
// halves), b likewise (high halves), for |a|, |b| above ~1e-33.  Each
// residual is exact in fp32 and has at most 16, then 8, significant bits.
__device__ __forceinline__ void split3_pk(float a, float b, unsigned& h, unsigned& m, unsigned& l) {
  h = pk_bf16(a, b);
  const float ra = a - __uint_as_float(h << 16), rb = b - __uint_as_float(h & 0xffff0000u);
  m = pk_bf16(ra, rb);
  const float sa = ra - __uint_as_float(m << 16), sb = rb - __uint_as_float(m & 0xffff0000u);
  l = pk_bf16(sa, sb);
}
// Eight floats split exactly into three bf16 terms, as MFMA operands.
__device__ __forceinline__ void split3_v8(const float (&v)[8], v8bf (&t)[3]) {
  v4u w[3];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    unsigned h, mm, l;
    split3_pk(v[2 * k], v[2 * k + 1], h, mm, l);
    w[0][k] = h;
    w[1][k] = mm;
    w[2][k] = l;
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) t[k] = __builtin_bit_cast(v8bf, w[k]);
}

__device__ __forceinline__ void ld8_bf16(const bf16_t* p, v4f& lo, v4f& hi) {
  const v4u w = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  lo[0] = __uint_as_float(w[0] << 16);
  lo[1] = __uint_as_float(w[0] & 0xffff0000u);
  lo[2] = __uint_as_float(w[1] << 16);
  lo[3] = __uint_as_float(w[1] & 0xffff0000u);
  hi[0] = __uint_as_float(w[2] << 16);
  hi[1] = __uint_as_float(w[2] & 0xffff0000u);
  hi[2] = __uint_as_float(w[3] << 16);
  hi[3] = __uint_as_float(w[3] & 0xffff0000u);
}
template <>
__device__ __forceinline__ v4f ld4_in<bf16_t>(const bf16_t* p) {
  const v2u w = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
  v4f r;
  r[0] = __uint_as_float(w[0] << 16);
  r[1] = __uint_as_float(w[0] & 0xffff0000u);
  r[2] = __uint_as_float(w[1] << 16);
  r[3] = __uint_as_float(w[1] & 0xffff0000u);
  return r;
}
// Buffer descriptor over `bytes` bytes at `base` (gfx9: 32-bit data format);
// accesses past the end are dropped by the hardware range check.
constexpr unsigned kBufWord3 = 0x00020000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufWord3);
}
// 16-byte store written through to memory (cache policy sc0 | sc1: system
// scope), leaving no dirty L2 line behind.
constexpr int kWriteThrough = 0x11;
__device__ __forceinline__ void st4_through(__amdgpu_buffer_rsrc_t rs, unsigned off, v4f v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), rs, off, 0, kWriteThrough);
}
// 16-byte store with the non-temporal hint (cache policy nt).
constexpr int kNonTemporal = 0x2;
__device__ __forceinline__ void st4_nt(__amdgpu_buffer_rsrc_t rs, unsigned off, v4f v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), rs, off, 0, kNonTemporal);
}

// Index of (sample smp in 0..15, state n in 0..15) inside a saved plane.  The
// backward lane (quad kg, state n) reads samples 4kg..4kg+3 as one float4.
__device__ __forceinline__ int plane_index(int smp, int n) { return (smp >> 2) * 64 + n * 4 + (smp & 3); }

// Planes saved per (16-sample block, state group): alpha'_t, beta'_t for the
// K steps, x_K, and one S_r per projection round when there is more than one.
__host__ __device__ __forceinline__ int saved_planes(int K) {
  const int rounds = (K + kChunk - 1) / kChunk;
  return 2 * K + 1 + (rounds > 1 ? rounds : 0);
}

// ---------------------------------------------------------------------------
// Forward.
//   grid  = 8 * NG * ceil(pairs * C / 8) work-groups (pairs: groups of one or
//   two sample blocks, C history chunks), 512 or 1024 threads each.
//   LDS   = 2 * SH2 * 16 * 3 * 2 B (weight terms) + 16 KiB (a|b exchange, also
//   the readout partials) + 2 KiB per wave (load tiles), per sample block.
// Work-group w runs on XCD w % 8; the NG state groups of one sample block are
// given consecutive rounds on the same XCD so their h_history reads share L2,
// and the chunks of a chunked history spread over the XCDs even when there
// are fewer sample blocks than XCDs.
//
// The weight slab is staged before any history load is issued (the vector
// memory pipe returns data in issue order, so slab loads queued behind the
// history stream would hold every MFMA back).  Each wave then keeps
// min(kFwdPrefetch, SH2/16) history loads in flight: enough in total to
// saturate HBM without queueing so deep that the first data arrives late.
// The first loads of round r+1 go out before the scan of round r.
// REPLAY (the second pass of a chunked history): the step projections a, b
// come from the alpha'/beta' slots, where the summary pass left them, instead
// of from h_history; only W_C is staged, for the readout.
// NBLK sample blocks per work-group: two for SH2 >= 320 (one work-group per
// CU, 16 waves), one when two-block work-groups would leave CUs idle (then
// 8 waves, with room for twice the loads in flight).
template <int NKC, class T, bool REPLAY = false, int NBLK = fwd_blocks(NKC)>  // SH2 / 16 trunk chunks;
// T = fp32 or bf16 trunk inputs
__global__ __launch_bounds__(NBLK * kFwdWaves * 64) void fwd_kernel(
    int B, int K, int NG, int NB,
    const T* __restrict__ H, const T* __restrict__ hs2,
    const float* __restrict__ WA, const float* __restrict__ WB, const float* __restrict__ WC,
    const float* __restrict__ stab, float* __restrict__ ctx, float* __restrict__ saved,
    int L, int C, int mode, const float* __restrict__ tw, float* __restrict__ he) {
  constexpr int SH2 = NKC * 16;
  constexpr int kFwdBlocks = NBLK;
  constexpr int kFwdThreads = NBLK * kFwdWaves * 64;
  constexpr bool kDeepSingle = NBLK == 1 && fwd_blocks(NKC) == 2;  // lone block of a wide trunk
  constexpr int NCR = (NKC + kFwdWaves - 1) / kFwdWaves;                   // readout chunks per wave
  constexpr int NCRP = (NKC / 2 + kFwdWaves - 1) / kFwdWaves;              // readout pairs per wave (bf16)
  // bf16 inputs come in pairs of chunks: lane (kg, m) holds features
  // 32p + 8kg .. +7 of pair p, the first four for chunk 2p, the rest for
  // chunk 2p+1 (the weight slab is staged in the same order).
  constexpr bool PAIR = sizeof(T) == 2;
  constexpr int PFP = PAIR ? (kDeepSingle ? 4 : (kFwdPairPrefetch < NKC / 2 ? kFwdPairPrefetch : NKC / 2))
                           : 0;  // loads in flight
  static_assert(!PAIR || PFP % 2 == 0, "bf16 loads go in spans of two pairs");
  // fp32 history on the bf16 matrix cores (SPL): each history value x is
  // split exactly into three bf16 terms as the weights w are (each term at
  // most 2^-8 of the one before), and six of the nine term products enter
  // the fp32 accumulator: the dropped mid*lo, lo*mid and lo*lo are below
  // 2^-23 of x*w together, about one fp32 rounding.  Per 32 features six
  // v_mfma_f32_16x16x32_bf16 replace eight v_mfma_f32_16x16x4_f32, about
  // 37 % of their matrix-core cycles at the two peaks; the split's
  // registers leave room for four loads in flight per wave.
  constexpr bool SPL = !PAIR && !REPLAY;
  constexpr int PF = PAIR ? 2 * PFP : (kDeepSingle ? 8 : (kFwdPrefetch < NKC ? kFwdPrefetch : NKC));  // in flight
  static_assert(PAIR || PF % 2 == 0, "fp32 loads go in pairs");
  // bf16 trunk inputs feed bf16 MFMAs directly: each weight is split
  // exactly into three bf16 terms (hi + mid + lo == W for every fp32 W above
  // ~1e-33), so every product is exact and only the fp32 accumulation
  // rounds, as with fp32 MFMAs.  The readout keeps fp32 MFMAs on widened
  // h_s2.
  constexpr bool BFM = PAIR && !REPLAY;
  constexpr bool WSPLIT = BFM || SPL;  // weights staged as three bf16 terms
  // History loads (CT): each load instruction covers 8 rows x 128 contiguous
  // bytes (lane (r8, p8): row r8 of one half of the block, 16 bytes at 16*p8
  // of a 128-byte span: 32 fp32 or 64 bf16 features), which streams ~10 %
  // faster than the MFMA operand order (16 rows x 64 B); the two halves of
  // a span go through a per-wave LDS tile into the operand order.  W_C then
  // comes straight from memory for the readout (its slab's LDS holds the
  // tiles).
  constexpr bool CT = !REPLAY;
  constexpr int NP = NKC / 2;  // 32-feature pairs of chunks
  __shared__ v4u sWab[WSPLIT ? 6 * NP * 64 : 1];  // [mat A|B][term hi|mid|lo][pair][lane]: 8 bf16
  __shared__ v4f sWc[CT ? 1 : NKC * 64];
  __shared__ v4f sT[CT ? kFwdBlocks * kFwdWaves * 128 : 1];  // CT: [wave][half j][64 slots]
  __shared__ __attribute__((aligned(16))) float sXa[kFwdBlocks][kChunk][kPlane];
  __shared__ __attribute__((aligned(16))) float sXb[kFwdBlocks][kChunk][kPlane];
  // readout partials; with BFM they share sXa's memory (summed into c
  // before the first exchange writes it), which keeps two work-groups per CU
  __shared__ __attribute__((aligned(16))) float sCbuf[WSPLIT ? 4 : kFwdBlocks * kFwdWaves * kPlane];
  float(*sC)[kFwdWaves][kPlane] = WSPLIT ? sXa : reinterpret_cast<float(*)[kFwdWaves][kPlane]>(sCbuf);

  const int D = NG * kGroup;
  const int xcd = blockIdx.x & 7;
  const int round = blockIdx.x >> 3;
  const int sg = round % NG;
  // (sample blocks, history chunk) items: without chunks (C = 1) they go
  // round-robin over the XCDs; with chunks each XCD takes a contiguous run of
  // items, so one block's chunks stay on few XCDs (128 samples, K = 2048:
  // summary pass 80.5 -> 79.3 us, K = 1024 with 64 samples 29.5 -> 28.3 us,
  // against dealing the chunks round-robin)
  const int item = C > 1 ? xcd * (int)(gridDim.x / (8 * NG)) + round / NG : (round / NG) * 8 + xcd;
  const int cidx = item % C;   // history chunk of this work-group
  const int pair = item / C;   // this work-group's sample blocks
  if (pair * kFwdBlocks >= NB) return;
  // steps [t0, t1) of this chunk: rounds r0 .. r1-1 (a round is kChunk steps)
  const int t0 = cidx * L;
  const int t1 = cidx == C - 1 ? K : t0 + L;
  const int r0 = t0 / kChunk;
  const int r1 = (t1 + kChunk - 1) / kChunk;

  const int tid = threadIdx.x;
  const int wg_wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar
  const int half = wg_wave / kFwdWaves;  // which of the work-group's blocks this wave serves
  const int wave = wg_wave % kFwdWaves;  // wave within its block
  const int lane = tid & 63;
  // The second block of the last pair may lie past NB: its waves take part
  // in every barrier but load a valid block (clamped) and store nothing.
  const bool blk_ok = pair * kFwdBlocks + half < NB;
  const int blk = min(pair * kFwdBlocks + half, NB - 1);
  const int kg = lane >> 4;  // k-group of the A/B operands, row quad of the result
  const int m = lane & 15;   // row of A (sample) / column of B and result (state)
  const int wlane = lane ^ ((lane >> 3) & 3);  // this lane's slot in a weight-slab pair (swizzled)

  // Scan lanes: waves 0..3, lane (i = lane>>4, n = lane&15) owns sample
  // smp = 4*wave + i and state n.
  const bool scanner = wave < 4 && blk_ok;
  const int smp = 4 * wave + kg;
  const int pidx = plane_index(smp & 15, m);
  // Saved planes of this (block, state group): alpha'_t and beta'_t for every
  // step, x_K, then, when K spans several rounds, S_r for every round r.
  const int nchunks = (K + kChunk - 1) / kChunk;  // rounds of the whole history
  const size_t blk_stride = (size_t)saved_planes(K) * kPlane;
  float* sv = saved + ((size_t)blk * NG + sg) * blk_stride;
  float x = 0.f, c = 0.f;
  // A chunked history (mode 2) starts from the state the carry pass left in
  // the chunk's second S plane, and scales its S_r by the product of every
  // later chunk's gates (the first S plane).  Read before anything is written.
  // The loads are unconditional (from the x_K plane, which always exists,
  // when not needed) and go out first, with the weight slab's: no wait on
  // them is computed from a branch or holds the history stream back.
  float suffix = 1.f;
  {
    const float x_in = sv[(size_t)(mode == 2 ? 2 * K + 2 + r0 : 2 * K) * kPlane + pidx];
    const float s_in = sv[(size_t)(mode == 2 ? 2 * K + 1 + r0 : 2 * K) * kPlane + pidx];
    const bool use = mode == 2 && scanner;
    x = use ? x_in : 0.f;
    suffix = use ? s_in : 1.f;
  }
  const float mstab = stab != nullptr ? stab[0] : 1.f;

  // (1) Weight slab, loaded before any history load is issued: the slab's
  // loads would otherwise queue behind the CU's history stream and hold every
  // MFMA back.  W_A and W_B go in as three bf16 terms each, in the
  // v_mfma_f32_16x16x32_bf16 B-operand layout; the replay pass stages only
  // W_C, in fp32 for the readout, where entry (kc, l) holds
  // W[kc*16 + 4*(l>>4) + i][sg*16 + (l&15)] for i = 0..3 (pair order for
  // bf16 inputs).
  // W_A, W_B (split terms): a task is (matrix, octet o of rows 8o..8o+7,
  // states 4*s4..4*s4+3), one per thread; per state n it writes the eight
  // rows' three terms as three 16-byte entries (pair o/4, lane (o%4, n)).
  // Entry l of a pair's 64 sits at slot wsw(l) = l ^ ((l >> 3) & 3): the
  // LDS serves a 16-byte access 8 lanes per cycle from 128 bytes of banks,
  // and with that swizzle both the staging writes (lanes 64 bytes apart)
  // and the operand reads (lane l reads entry l) touch 8 distinct 16-byte
  // bank groups per 8 lanes.
  // The rows are loaded here and waited for; the split and its LDS writes
  // run after the first history loads have gone out, under their latency.
  constexpr int NTASK = 2 * (SH2 / 8) * 4;  // = SH2
  static_assert(!WSPLIT || NTASK <= kFwdThreads, "one weight task per thread");
  const int w_mat = tid / ((SH2 / 8) * 4);
  const int w_o = (tid >> 2) % (SH2 / 8);
  const int w_s4 = tid & 3;
  v4f wst[WSPLIT ? 8 : 1];
  if constexpr (WSPLIT) {
    if (tid < NTASK) {
      const float* W = w_mat == 0 ? WA : WB;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) wst[jj] = ld4(W + (size_t)(8 * w_o + jj) * D + sg * kGroup + 4 * w_s4);
      __asm__ volatile("" ::"v"(wst[7][0]));  // wait for the rows (they return in order)
    }
  }
  auto stage_split = [&]() {
    if (tid < NTASK) {
      const int mat = w_mat, o = w_o, s4 = w_s4;
      const v4f* w = wst;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v8bf th, tm, tl;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float v = w[jj][q];
          const __bf16 hi = (__bf16)v;
          const float r1 = v - (float)hi;
          const __bf16 mi = (__bf16)r1;
          const float r2 = r1 - (float)mi;
          th[jj] = hi;
          tm[jj] = mi;
          tl[jj] = (__bf16)r2;
        }
        const int el = (o & 3) * 16 + 4 * s4 + q;  // entry within the pair
        const int e = (o >> 2) * 64 + (el ^ ((el >> 3) & 3));
        sWab[(mat * 3 + 0) * NP * 64 + e] = __builtin_bit_cast(v4u, th);
        sWab[(mat * 3 + 1) * NP * 64 + e] = __builtin_bit_cast(v4u, tm);
        sWab[(mat * 3 + 2) * NP * 64 + e] = __builtin_bit_cast(v4u, tl);
      }
    }
  };
  if constexpr (!WSPLIT) {
    // REPLAY: only W_C, for the readout
    constexpr int NW4 = SH2 * 4;  // float4s of the slab
    constexpr int NWT = (NW4 + kFwdThreads - 1) / kFwdThreads;
    v4f wr[NWT];
#pragma unroll
    for (int it = 0; it < NWT; ++it) {
      const int r = tid + it * kFwdThreads;
      if (r < NW4) wr[it] = ld4(WC + (size_t)(r >> 2) * D + sg * kGroup + 4 * (r & 3));
    }
#pragma unroll
    for (int it = 0; it < NWT; ++it) {
      const int r = tid + it * kFwdThreads;
      if (r < NW4) {
        const int j = r >> 2, s4 = r & 3;
        float* dst = reinterpret_cast<float*>(sWc);
        // feature j -> (chunk, k-group, element) of the A/B operand order
        const int jc = PAIR ? 2 * (j >> 5) + ((j & 7) >> 2) : (j >> 4);
        const int jg = PAIR ? ((j & 31) >> 3) : ((j >> 2) & 3);
        const int base = (jc * 64 + 16 * jg + 4 * s4) * 4 + (j & 3);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[base + 4 * q] = wr[it][q];
      }
    }
  }
  __syncthreads();

  // (2) A-operand row of this lane: sample blk*16 + m, clamped into range
  // (rows of samples >= B are computed but never stored and never reach a
  // gradient).  Readout chunks kc = wave + 8r, then this wave's first step:
  // all issued now, consumed by the MFMAs below as they land.
  const int smp_a = min(blk * kBlock + m, B - 1);
  const int koff = PAIR ? 8 * kg : 4 * kg;
  const T* crow = hs2 + (size_t)smp_a * SH2 + koff;
  v4f hc[PAIR ? 2 * NCRP : NCR];
  if constexpr (PAIR) {
#pragma unroll
    for (int r = 0; r < NCRP; ++r) {
      const int pc = min(wave + kFwdWaves * r, NKC / 2 - 1);
      ld8_bf16(crow + pc * 32, hc[2 * r], hc[2 * r + 1]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < NCR; ++r) {
      const int kc = min(wave + kFwdWaves * r, NKC - 1);
      hc[r] = ld4_in(crow + kc * 16);
    }
  }
  // CT: the readout's W_C operand, W_C[f + i][sg*16 + m] for the features
  // f + i (i = 0..3) that this lane's h_s2 values carry
  v4f wcv[CT ? (PAIR ? 2 * NCRP : NCR) : 1];
  if constexpr (CT && PAIR) {
#pragma unroll
    for (int r = 0; r < NCRP; ++r) {
      const int pc = min(wave + kFwdWaves * r, NKC / 2 - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wcv[2 * r + h][i] = WC[(size_t)(pc * 32 + 8 * kg + 4 * h + i) * D + sg * kGroup + m];
    }
  } else if constexpr (CT) {
#pragma unroll
    for (int r = 0; r < NCR; ++r) {
      const int kc = min(wave + kFwdWaves * r, NKC - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) wcv[r][i] = WC[(size_t)(kc * 16 + 4 * kg + i) * D + sg * kGroup + m];
    }
  }
  // CT: lane (r8, p8) loads rows r8 and 8 + r8 of the block
  const int r8 = lane >> 3, p8 = lane & 7;
  const T* hb0 = H + (size_t)min(blk * kBlock + r8, B - 1) * K * SH2 + (16 / sizeof(T)) * p8;
  const T* hb1 = H + (size_t)min(blk * kBlock + 8 + r8, B - 1) * K * SH2 + (16 / sizeof(T)) * p8;
  v4f hv[BFM ? 1 : NKC];
  v4u hr[BFM ? NP : 1];  // BFM: raw bf16 pairs
  // chunk kc (or pair kc/2) of history step t into hv (or hr)
  auto load_chunk = [&](int t, int kc) {
    if constexpr (BFM)  // load kc/2: half (kc/2) & 1 of the 64-feature span kc/4
      hr[kc >> 1] = __builtin_nontemporal_load(
          reinterpret_cast<const v4u*>((((kc >> 1) & 1) ? hb1 : hb0) + (size_t)t * SH2 + (kc >> 2) * 64));
    else  // fp32, load kc: half kc & 1 of pair kc >> 1
      hv[kc] = ld4_in(((kc & 1) ? hb1 : hb0) + (size_t)t * SH2 + (kc >> 1) * 32);
  };
  // CT tile slots (16 bytes each), XOR-swizzled so that the writes of 8
  // lanes and the operand reads of 16 lanes each touch distinct banks: lane
  // (r8, p8) of half j writes slot 64j + 8r8 + (p8 ^ r8 ^ j); operand lane
  // (kg, m) of half-span h (fp32: chunk h of the pair; bf16: pair h of the
  // span) reads row m's 16 bytes at 16*(4h + kg).
  v4f* tile = sT + (CT ? wg_wave * 128 : 0);
  const int wslot0 = 8 * r8 + (p8 ^ r8);
  const int wslot1 = 64 + 8 * r8 + (p8 ^ r8 ^ 1);
  const int rslot0 = 64 * (m >> 3) + 8 * (m & 7) + ((0 + kg) ^ (m & 7) ^ (m >> 3));
  const int rslot1 = 64 * (m >> 3) + 8 * (m & 7) + ((4 + kg) ^ (m & 7) ^ (m >> 3));
  // fp32: operand lane (kg, m) reads row m's 32 bytes at 32*kg (slots 2kg
  // and 2kg + 1, which differ in the last bit after the swizzle as well)
  const int rslot8 = 64 * (m >> 3) + 8 * (m & 7) + ((2 * kg) ^ (m & 7) ^ (m >> 3));
  // REPLAY: this wave's step projections, as float4s of the alpha'/beta'
  // slots (its four samples 4kg+r at state m are entries kg*64 + 4m + r,
  // the MFMA result layout)
  const int toff = kg * 64 + 4 * m;
  v4f pa = {0.f, 0.f, 0.f, 0.f}, pb = {0.f, 0.f, 0.f, 0.f};
  {
    // a wave past the chunk's last step loads that step again (unused)
    const int tf = min(t0 + wave, t1 - 1);
    if constexpr (REPLAY) {
      pa = ld4(sv + (size_t)(2 * tf) * kPlane + toff);
      pb = ld4(sv + (size_t)(2 * tf + 1) * kPlane + toff);
    } else {
#pragma unroll
      for (int kc = 0; kc < PF; kc += PAIR ? 2 : 1) load_chunk(tf, kc);
    }
  }
  // keep these loads here, ahead of the readout (the compiler would
  // otherwise sink them to their first use)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (WSPLIT) stage_split();  // read after the barrier below

  // (3) readout partial over this wave's chunks (a clamped chunk past the
  // last one enters as zeros: no branch, so no load is moved under one)
  {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (PAIR) {
#pragma unroll
      for (int r = 0; r < NCRP; ++r) {
        const int pc = wave + kFwdWaves * r;
        const bool ok = pc < NKC / 2;
        const int pcc = min(pc, NKC / 2 - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          v4f bv;
          if constexpr (CT)
            bv = wcv[2 * r + h];
          else
            bv = sWc[(2 * pcc + h) * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc = mfma16x16x4(ok ? hc[2 * r + h][i] : 0.f, bv[i], acc);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < NCR; ++r) {
        const int kc = wave + kFwdWaves * r;
        const bool ok = kc < NKC;
        v4f bv;
        if constexpr (CT)
          bv = wcv[r];
        else
          bv = sWc[min(kc, NKC - 1) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mfma16x16x4(ok ? hc[r][i] : 0.f, bv[i], acc);
      }
    }
    // result rows 4kg..4kg+3 at state m: one float4 in the plane layout
    *reinterpret_cast<v4f*>(&sC[half][wave][kg * 64 + 4 * m]) = acc;
  }
  if constexpr (WSPLIT) {
    // sum the readout now: the partials' memory is sXa's
    __syncthreads();
    if (scanner) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kFwdWaves; ++w) s += sC[half][w][plane_index(smp, m)];
      c = s;
    }
    __syncthreads();
  }

  float G[kChunk];
  float Gr[kRegRounds];  // gate product of each round (rounds >= kRegRounds park theirs in saved)
#pragma unroll
  for (int i = 0; i < kRegRounds; ++i) Gr[i] = 1.f;

  float gq[4] = {0.f, 0.f, 0.f, 0.f};  // this wave's step: m g (1 - g), for alpha'_t
  // Rounds r0 .. r1-1 of this chunk: at least one (a chunk is never empty),
  // written as do-while so the first round's loads above stay where they
  // are issued instead of moving into a loop-entry test.
  int ch = r0;
  do {
    const int lr = ch - r0;  // round within this chunk
    const int t = ch * kChunk + wave;
    v4f sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};  // this step's projections
    if (t < t1) {
      v4f acca = {0.f, 0.f, 0.f, 0.f};
      v4f accb = {0.f, 0.f, 0.f, 0.f};
      if constexpr (REPLAY) {
        acca = pa;
        accb = pb;
        // the next round's projections go out now
        if (t + kChunk < t1) {
          pa = ld4(sv + (size_t)(2 * (t + kChunk)) * kPlane + toff);
          pb = ld4(sv + (size_t)(2 * (t + kChunk) + 1) * kPlane + toff);
        }
      } else if constexpr (BFM) {
#pragma unroll
      for (int q4 = 0; q4 < NP / 2; ++q4) {
        // the span's two loads into this wave's tile, then back as the
        // operands of pairs 2*q4 and 2*q4 + 1
        tile[wslot0] = __builtin_bit_cast(v4f, hr[2 * q4]);
        tile[wslot1] = __builtin_bit_cast(v4f, hr[2 * q4 + 1]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const v4f h0 = tile[rslot0];
        const v4f h1 = tile[rslot1];
        // keep PFP loads of this step in flight
        if (2 * q4 + PFP < NP) load_chunk(t, 2 * (2 * q4 + PFP));
        if (2 * q4 + 1 + PFP < NP) load_chunk(t, 2 * (2 * q4 + 1 + PFP));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int pp = 2 * q4 + hh;
          const v8bf h = __builtin_bit_cast(v8bf, hh ? h1 : h0);
#pragma unroll
          for (int tm = 0; tm < 3; ++tm) {
            acca = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                h, __builtin_bit_cast(v8bf, sWab[(0 * 3 + tm) * NP * 64 + pp * 64 + wlane]), acca, 0, 0, 0);
            accb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                h, __builtin_bit_cast(v8bf, sWab[(1 * 3 + tm) * NP * 64 + pp * 64 + wlane]), accb, 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // next round's first loads go out before this round's exchange and scan
      if (t + kChunk < t1) {
#pragma unroll
        for (int kc = 0; kc < PF; kc += 2) load_chunk(t + kChunk, kc);
      }
      } else {  // fp32 history, split into bf16 terms
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        // the pair's two loads into this wave's tile, then back as this
        // lane's eight consecutive features 32pp + 8kg .. +7 of row m
        tile[wslot0] = hv[2 * pp];
        tile[wslot1] = hv[2 * pp + 1];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // keep PF loads of this step in flight
        if (2 * pp + PF < NKC) load_chunk(t, 2 * pp + PF);
        if (2 * pp + 1 + PF < NKC) load_chunk(t, 2 * pp + 1 + PF);
        v4u xw[3];  // the three terms, two bf16 per word
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const v4f x = tile[rslot8 ^ hf];
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            unsigned h, mm, l;
            split3_pk(x[2 * w], x[2 * w + 1], h, mm, l);
            xw[0][2 * hf + w] = h;
            xw[1][2 * hf + w] = mm;
            xw[2][2 * hf + w] = l;
          }
        }
        v8bf xt[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) xt[k] = __builtin_bit_cast(v8bf, xw[k]);
        // weight term tw with history terms ta <= 2 - tw, the smaller
        // products first; one weight term's operands live at a time
#pragma unroll
        for (int tw = 2; tw >= 0; --tw) {
          const v8bf wa = __builtin_bit_cast(v8bf, sWab[(0 * 3 + tw) * NP * 64 + pp * 64 + wlane]);
          const v8bf wb = __builtin_bit_cast(v8bf, sWab[(1 * 3 + tw) * NP * 64 + pp * 64 + wlane]);
#pragma unroll
          for (int ta = 2 - tw; ta >= 0; --ta) {
            acca = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xt[ta], wa, acca, 0, 0, 0);
            accb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xt[ta], wb, accb, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // next round's first loads go out before this round's exchange and scan
      if (t + kChunk < t1) {
#pragma unroll
        for (int kc = 0; kc < PF; ++kc) load_chunk(t + kChunk, kc);
      }
      }
      sa = acca;
      sb = accb;
      __builtin_amdgcn_sched_barrier(0);
      // The gates of this step, for this lane's four samples (rows 4kg+r):
      // sigmoid(a) = 1 / (1 + e^-a) from the hardware exp2 and reciprocal
      // (each within ~1 ulp); e = inf gives g = 0, never NaN.  1 - g is
      // computed without cancellation: e*g = e/(1+e) for a > 0.  The
      // stability multiplier m scales the gate and its derivative (m = 1
      // leaves every product bit-identical).  The exchange carries m*g and b;
      // m g (1 - g) stays here for this step's alpha' below.
      v4f mg;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = acca[r];
        const float e = __expf(-a);
        const float g = __builtin_amdgcn_rcpf(1.f + e);
        gq[r] = g * (a > 0.f ? e * g : 1.f - g) * mstab;
        mg[r] = g * mstab;
      }
      // the exchange holds tiles in the plane layout: this lane's four
      // samples 4kg..4kg+3 at state m are one float4
      *reinterpret_cast<v4f*>(&sXa[half][wave][kg * 64 + 4 * m]) = mg;
      *reinterpret_cast<v4f*>(&sXb[half][wave][kg * 64 + 4 * m]) = accb;
    }
    __syncthreads();

    if (scanner) {
      const int idx = plane_index(smp, m);
      if (!WSPLIT && ch == r0) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kFwdWaves; ++w) s += sC[half][w][idx];
        c = s;
      }
      const int tn = min(kChunk, t1 - ch * kChunk);
      // The recurrence; each step's slot then holds the state it started
      // from (x_t), for the projecting wave's alpha'.
#pragma unroll
      for (int tt = 0; tt < kChunk; ++tt) {
        if (tt < tn) {
          G[tt] = sXa[half][tt][idx];
          const float b = sXb[half][tt][idx];
          sXa[half][tt][idx] = x;
          x = G[tt] * x + b;
        }
      }
      // Round-local reverse pass: beta'_t = c * prod of this round's later
      // gates (into the step's second slot), and the round's gate product.
      // The full terms are beta_t = S_r beta'_t and alpha_t = S_r alpha'_t
      // with S_r the product of every gate of the later rounds; the backward
      // applies S_r.
      float P = c, gp = 1.f;
#pragma unroll
      for (int tt = kChunk - 1; tt >= 0; --tt) {
        if (tt < tn) {
          sXb[half][tt][idx] = P;
          P *= G[tt];
          gp *= G[tt];
        }
      }
      if (nchunks > 1) {
        if (lr < kRegRounds) {
#pragma unroll
          for (int i = 0; i < kRegRounds; ++i)
            if (i == lr) Gr[i] = gp;
        } else {
          sv[(size_t)(2 * K + 1 + ch) * kPlane + pidx] = gp;  // read back below, same thread
        }
      }
    }
    __syncthreads();
    // Each projecting wave writes its step's planes: beta'_t and
    // alpha'_t = beta'_t * x_t * m g (1 - g), one float4 per lane (its four
    // samples 4kg+r at state m are entries kg*64 + 4m + r of a plane).  The
    // stores are unconditional; a descriptor of size 0 drops them for a wave
    // past the chunk's last step (and in the summary pass), so no memory
    // operation sits under a branch while the next round's loads are in
    // flight.  (Every wave reads back only its own slots here, and writes
    // them again only after its next projection, so no barrier is needed
    // within the rounds; whatever writes these slots after the last round
    // -- the fused blend below -- waits at a barrier first.)
    {
      const bool st_ok = t < t1 && blk_ok;
      const int ts = min(t, t1 - 1);
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(sv + (size_t)(2 * ts) * kPlane, st_ok ? 2 * kPlane * sizeof(float) : 0u);
      v4f al, be;
      const v4f xq = *reinterpret_cast<const v4f*>(&sXa[half][wave][kg * 64 + 4 * m]);
      const v4f pq = *reinterpret_cast<const v4f*>(&sXb[half][wave][kg * 64 + 4 * m]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        al[r] = pq[r] * (xq[r] * gq[r]);
        be[r] = pq[r];
      }
      const unsigned off = (unsigned)(toff * sizeof(float));
      st4_nt(rs, off, mode == 1 ? sa : al);
      st4_nt(rs, off + kPlane * sizeof(float), mode == 1 ? sb : be);
    }
  } while (++ch < r1);

  // The h_enriched blend (one state group: every state of these samples is
  // here): he[b][j] = h_s2[b][j] + w_j * (sum_s context[b][s]) / D, by the
  // work-group that writes context.  The h_s2 rows are read again here
  // rather than kept in registers through the rounds.
  if constexpr (!PAIR) {
    if (he != nullptr && NG == 1 && cidx == C - 1) {  // uniform over the work-group
      // sC[half][0] is wave 0's exchange slot when the weights are split
      // (sC aliases sXa): wave 0 may still be reading it for its last
      // alpha' store above, so every wave passes this barrier before the
      // scanners overwrite it.
      __syncthreads();
      if (scanner) sC[half][0][plane_index(smp, m)] = c * x;
      __syncthreads();
      float sum = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < kGroup; ++s2) sum += sC[half][0][plane_index(m, s2)];  // states in order
      const float scale = sum * (1.f / (float)kGroup);                         // exact: D = 16
      const int b_row = blk * kBlock + m;
#pragma unroll
      for (int r = 0; r < NCR; ++r) {
        const int kc = wave + kFwdWaves * r;
        if (kc < NKC && b_row < B && blk_ok) {
          const int f0 = kc * 16 + 4 * kg;
          const v4f wv = tw != nullptr ? ld4(tw + f0) : v4f{1.f, 1.f, 1.f, 1.f};
          const v4f hv2 = ld4_stream(hs2 + (size_t)b_row * SH2 + f0);
          v4f o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = hv2[q] + wv[q] * scale;
          __builtin_nontemporal_store(o, reinterpret_cast<v4f*>(he + (size_t)b_row * SH2 + f0));
        }
      }
    }
  }

  if (!scanner) return;

  if (mode == 1) {
    // summary of this chunk for the carry pass: the product of its gates
    // (first S plane) and its final state from x = 0 (second S plane)
    float G_all = 1.f;
    for (int ch = r0; ch < r1; ++ch) {
      const int lr = ch - r0;
      float g = 1.f;
      if (lr < kRegRounds) {
#pragma unroll
        for (int i = 0; i < kRegRounds; ++i)
          if (i == lr) g = Gr[i];
      } else {
        g = sv[(size_t)(2 * K + 1 + ch) * kPlane + pidx];
      }
      G_all *= g;
    }
    sv[(size_t)(2 * K + 1 + r0) * kPlane + pidx] = G_all;
    sv[(size_t)(2 * K + 2 + r0) * kPlane + pidx] = x;
    return;
  }

  if (cidx == C - 1) {
    const int b_glob = blk * kBlock + smp;
    if (b_glob < B) st_stream(&ctx[(size_t)b_glob * D + sg * kGroup + m], c * x);
    st_stream(&sv[(size_t)(2 * K) * kPlane + pidx], x);
  }

  // S_r = product of the gates of rounds r+1 .. last (S_last = 1): this
  // chunk's later rounds, times every later chunk's gates.
  if (nchunks > 1) {
    float S = suffix;
    for (int ch = r1 - 1; ch >= r0; --ch) {
      const int lr = ch - r0;
      float* ps = &sv[(size_t)(2 * K + 1 + ch) * kPlane + pidx];
      float g = 1.f;
      if (lr < kRegRounds) {
#pragma unroll
        for (int i = 0; i < kRegRounds; ++i)
          if (i == lr) g = Gr[i];
      } else {
        g = *ps;
      }
      st_stream(ps, S);
      S *= g;
    }
  }
}

// Carry across the chunks of a chunked history, per (sample, state) entry
// of a (block, state group): from each chunk's summary (G_c = product of its
// gates, X_c = its final state from 0; first and second S plane of its first
// round) to the state it starts from,
//   x_start(0) = 0,  x_start(c+1) = G_c x_start(c) + X_c,
// (second S plane) and the product of every later chunk's gates (first).
// The chunks of an entry are cut into T segments of at most kCarrySeg
// consecutive chunks, one thread each, all of a segment's summaries loaded
// at once.  A segment composes to one affine map (product of its gates, its
// state from 0); each thread then composes the maps of the segments before
// its own (from LDS) for its start state and multiplies the gate products of
// the segments after it, and walks its chunks once forward and once back.
// Work-group (bg, part): 256 threads, entries part*256/T .. +256/T - 1 of
// (block, state group) bg, T segments each (T a power of two, <= 32).
constexpr int kCarrySeg = 16;
constexpr int kCarryThreads = 256;

static_assert(kFwdChunkTarget / kCarrySeg <= kCarryThreads, "carry segments per entry fit a work-group");

int carry_segments(int C) {
  int t = 1;
  while (t * kCarrySeg < C) t *= 2;
  return t;
}

__global__ __launch_bounds__(kCarryThreads) void fwd_carry_kernel(int NBG, int K, int L, int C, int T,
                                                                  float* __restrict__ saved) {
  __shared__ float sG[kCarryThreads], sX[kCarryThreads];  // [segment][entry of the work-group]
  const int epg = kCarryThreads / T;  // entries per work-group
  const int bg = blockIdx.x / T;      // (block, state group)
  if (bg >= NBG) return;
  const int j = threadIdx.x / epg;    // segment
  const int el = threadIdx.x % epg;
  const int e = (blockIdx.x % T) * epg + el;  // entry of the 16 x 16 plane
  float* sv = saved + (size_t)bg * saved_planes(K) * kPlane + e;
  const int rpc = L / kChunk;  // rounds per chunk
  auto gate = [&](int cc) { return sv + (size_t)(2 * K + 1 + cc * rpc) * kPlane; };
  auto state = [&](int cc) { return sv + (size_t)(2 * K + 2 + cc * rpc) * kPlane; };
  const int M = (C + T - 1) / T;  // chunks per segment, <= kCarrySeg
  const int c0 = j * M;
  const int n = max(0, min(C, c0 + M) - c0);  // this segment's chunks (the last may be short or empty)
  float G[kCarrySeg], X[kCarrySeg];
#pragma unroll
  for (int i = 0; i < kCarrySeg; ++i) {  // clamped: every load unconditional
    const int cc = min(c0 + min(i, n - 1), C - 1);
    G[i] = *gate(max(cc, 0));
    X[i] = *state(max(cc, 0));
  }
  float gs = 1.f, xs = 0.f;  // the segment's map: x -> gs x + xs
#pragma unroll
  for (int i = 0; i < kCarrySeg; ++i) {
    if (i < n) {
      xs = G[i] * xs + X[i];
      gs *= G[i];
    }
  }
  sG[threadIdx.x] = gs;
  sX[threadIdx.x] = xs;
  __syncthreads();
  float x = 0.f, S = 1.f;
  for (int jj = 0; jj < T; ++jj) {
    const float g = sG[jj * epg + el], xx = sX[jj * epg + el];
    if (jj < j) x = g * x + xx;
    if (jj > j) S *= g;
  }
#pragma unroll
  for (int i = 0; i < kCarrySeg; ++i) {
    if (i < n) {
      *state(c0 + i) = x;
      x = G[i] * x + X[i];
    }
  }
#pragma unroll
  for (int i = kCarrySeg - 1; i >= 0; --i) {
    if (i < n) {
      *gate(c0 + i) = S;
      S *= G[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, phase 1: split-K partial products.
//   grid = 8 * V * ceil(P / 8), V = (SH2/64) * NG variants, 768 threads
//   (12 waves: three per SIMD, for the matrix cores to have work while
//   other waves wait for memory); 512 threads with paired steps (below),
//   whose units hold twice the registers.
// Work-group w: XCD w % 8, variant v = (w/8) % V (column block jb, state
// group sg), slice p = ((w/8) / V) * 8 + w % 8 covering units
// [p*UPW, min(NB*(K+1), (p+1)*UPW)), unit u = (block u / (K+1), step u % (K+1)),
// so a long history with few samples still spreads over many work-groups.
//
// MFMA roles (v_mfma_f32_16x16x4_f32, D[M=16][N=16] += A[16][4] B[4][16]):
//   M = features jb*64 + 4*row + q (four M tiles q share one float4 load),
//   N = states sg*16 + n, K = the 4 samples 4*kg + i of step i.
//   A lane (kg, m): H[sample 4kg+i][t][jb*64 + 4m + q]
//   B lane (kg, n): d_x[sample 4kg+i][t][n]
//
// Units: each sample block contributes K "step" units (H^T [d_a|d_b] at one
// history step) and one "readout" unit (h_s2^T d_c).  Wave w takes units
// w, w+12, ... (so the waves of a work-group read neighbouring rows at the
// same time); each wave keeps the loads of its next unit in flight while it
// multiplies the current one.  The unit index is scalar (the wave index is
// read as a scalar), so block, step and row bases cost scalar instructions
// only.
struct BwdUnit {
  v4f h[4];   // A operands: 4 rows (samples 4kg+i) x 4 features
  v2u hr[4];  // bf16 inputs: the same, as loaded (four bf16 per row)
  v4f al;     // alpha'_t (step unit) or x_K (readout unit), samples 4kg..4kg+3
  v4f be;     // beta'_t (step unit)
  v4f sr;     // S_r of the step's round (1 when K fits one round)
  float dc[4];  // d_context of samples 4kg+i, state n (unmasked)
  int blk, t, nvalid;  // the unit's block and step (t == K: readout), samples below B
};

// Per-work-group constants, and this lane's fixed offsets.  The unit index is
// the same for every lane of a wave, so everything that depends only on it
// (block, step, plane, row bases) is scalar arithmetic; a lane adds its own
// sample row (4kg), feature column and state.
template <class T>
struct BwdCtx {
  int B, K, SH2, D, NG, sg, u0, kg, state;
  int UPB;  // units per sample block: K steps (or ceil(K/2) step pairs) and the readout
  const T* H;
  const T* hs2;
  const float* saved;
  const float* dctx;
  size_t blk_stride;
  bool rounds;  // K spans more than one round: apply S_r
  long long hk_step, hk_out;  // elements from a unit's row i to row 4kg+i: step rows, readout rows
  int col;                    // jb*64 + 4m: first of this lane's four features
};


// Every unit issues the same loads, from addresses chosen by select: a step
// unit reads alpha'_t, beta'_t, S_r (ROUNDS: K spans several rounds) and
// four H rows; the readout reads x_K (in each plane's place) and four h_s2
// rows.  With no memory operation under a branch
// the compiler's memory-counter waits stay exact, so the next unit's loads
// (issued before this unit is consumed) stay in flight.  Rows of samples past
// B (last block only) re-read a valid row; their d_context is masked to zero.
template <bool ROUNDS, class T>
__device__ __forceinline__ void bwd_load(BwdUnit& U, int u, const BwdCtx<T>& c, int lane) {
  // unit u of the work-group's slice: block and step (t == K: the readout)
  const int ug = c.u0 + u;
  BwdUnit& q = U;
  q.blk = ug / c.UPB;
  q.t = ug - q.blk * c.UPB;
  q.nvalid = c.B - q.blk * kBlock;
  const bool step = q.t < c.K;
  const float* sv = c.saved + ((size_t)q.blk * c.NG + c.sg) * c.blk_stride;
  const int p0 = step ? 2 * q.t : 2 * c.K;
  const int p1 = step ? 2 * q.t + 1 : 2 * c.K;
  U.al = ld4(sv + (size_t)p0 * kPlane + 4 * lane);
  U.be = ld4(sv + (size_t)p1 * kPlane + 4 * lane);
  if constexpr (ROUNDS) {
    const int ps = step ? 2 * c.K + 1 + q.t / kChunk : 2 * c.K;  // a valid plane either way
    U.sr = ld4(sv + (size_t)ps * kPlane + 4 * lane);
  }
  const T* rows = step ? c.H + (size_t)q.t * c.SH2 : c.hs2;
  const size_t rstride = step ? (size_t)c.K * c.SH2 : (size_t)c.SH2;  // elements between samples
  const long long hk = step ? c.hk_step : c.hk_out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s0 = min(q.blk * kBlock + i, c.B - 1);  // row i of the block (scalar)
    const bool ok = 4 * c.kg + i < q.nvalid;
    const T* hp = rows + (size_t)s0 * rstride + (ok ? hk : 0) + c.col;
    if constexpr (sizeof(T) == 2)
      U.hr[i] = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(hp));
    else
      U.h[i] = ld4_in(hp);
    U.dc[i] = c.dctx[(size_t)s0 * c.D + (ok ? 4 * c.kg * c.D : 0) + c.state];
  }
}

// DBG: also store d_a, d_b, d_c (a separate instantiation, so the product
// path carries no stores and no branches for them).
// bf16 history: one v_mfma_f32_16x16x16_bf16 per tile and term covers all
// 16 samples of the unit.  Its A operand (feature 4m+q, samples 4kg..4kg+3)
// is gathered from the four rows this lane loaded; its B operand is d split
// exactly into three bf16 terms, so every product is exact and only the
// fp32 accumulation rounds.
__device__ __forceinline__ void bf16_split3(const float (&d)[4], v4bf (&t)[3]) {
  unsigned h0, m0, l0, h1, m1, l1;
  split3_pk(d[0], d[1], h0, m0, l0);
  split3_pk(d[2], d[3], h1, m1, l1);
  t[0] = __builtin_bit_cast(v4bf, v2u{h0, h1});
  t[1] = __builtin_bit_cast(v4bf, v2u{m0, m1});
  t[2] = __builtin_bit_cast(v4bf, v2u{l0, l1});
}
__device__ __forceinline__ void bf16_tiles(const BwdUnit& U, v4bf (&a)[4]) {
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    // the low (qq even) or high (qq odd) halves of two rows' words, row 0's
    // in the low half of the result (one byte permute)
    const int w = qq >> 1;
    const unsigned sel = (qq & 1) ? 0x07060302u : 0x05040100u;
    v2u p;
    p[0] = __builtin_amdgcn_perm(U.hr[1][w], U.hr[0][w], sel);
    p[1] = __builtin_amdgcn_perm(U.hr[3][w], U.hr[2][w], sel);
    a[qq] = __builtin_bit_cast(v4bf, p);
  }
}

// dv (when the caller keeps it): the unit's d values as this lane holds
// them, samples 4kg..4kg+3 of state n: [0] d_a or d_c, [1] d_b.
template <bool DBG, bool ROUNDS, bool BF, class Ctx>
__device__ __forceinline__ void bwd_compute(const BwdUnit& U, bool live, const Ctx& c, v4f (&acc)[4][3],
                                            float* __restrict__ d_a_out, float* __restrict__ d_b_out,
                                            float* __restrict__ d_c_out, bool write_dbg, float (&dv)[2][4]) {
  const BwdUnit& q = U;
  const int sbase = q.blk * kBlock + 4 * c.kg;
  if constexpr (BF) {
    v4bf a[4];
    bf16_tiles(U, a);
    if (q.t < c.K) {
      float da[4], db[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = live && 4 * c.kg + i < q.nvalid;
        const float dc = ok ? (ROUNDS ? U.dc[i] * U.sr[i] : U.dc[i]) : 0.f;
        da[i] = dc * U.al[i];
        db[i] = dc * U.be[i];
        if (DBG && write_dbg && ok) {
          const int s = sbase + i;
          if (d_a_out) d_a_out[((size_t)s * c.K + q.t) * c.D + c.state] = da[i];
          if (d_b_out) d_b_out[((size_t)s * c.K + q.t) * c.D + c.state] = db[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dv[0][i] = da[i];
        dv[1][i] = db[i];
      }
      v4bf ta[3], tb[3];
      bf16_split3(da, ta);
      bf16_split3(db, tb);
#pragma unroll
      for (int tm = 0; tm < 3; ++tm)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          acc[qq][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[qq], ta[tm], acc[qq][0], 0, 0, 0);
          acc[qq][1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[qq], tb[tm], acc[qq][1], 0, 0, 0);
        }
    } else {
      float dd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = live && 4 * c.kg + i < q.nvalid;
        dd[i] = (ok ? U.dc[i] : 0.f) * U.al[i];
        if (DBG && write_dbg && ok && d_c_out) d_c_out[(size_t)(sbase + i) * c.D + c.state] = dd[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) dv[0][i] = dd[i];
      v4bf td[3];
      bf16_split3(dd, td);
#pragma unroll
      for (int tm = 0; tm < 3; ++tm)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          acc[qq][2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[qq], td[tm], acc[qq][2], 0, 0, 0);
    }
    return;
  }
  if (q.t < c.K) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = live && 4 * c.kg + i < q.nvalid;
      const float dc = ok ? (ROUNDS ? U.dc[i] * U.sr[i] : U.dc[i]) : 0.f;
      const float da = dc * U.al[i];
      const float db = dc * U.be[i];
      dv[0][i] = da;
      dv[1][i] = db;
      if (DBG && write_dbg && ok) {
        const int s = sbase + i;
        if (d_a_out) d_a_out[((size_t)s * c.K + q.t) * c.D + c.state] = da;
        if (d_b_out) d_b_out[((size_t)s * c.K + q.t) * c.D + c.state] = db;
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        acc[qq][0] = mfma16x16x4(U.h[i][qq], da, acc[qq][0]);
        acc[qq][1] = mfma16x16x4(U.h[i][qq], db, acc[qq][1]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = live && 4 * c.kg + i < q.nvalid;
      const float dcc = (ok ? U.dc[i] : 0.f) * U.al[i];
      dv[0][i] = dcc;
      if (DBG && write_dbg && ok && d_c_out) d_c_out[(size_t)(sbase + i) * c.D + c.state] = dcc;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) acc[qq][2] = mfma16x16x4(U.h[i][qq], dcc, acc[qq][2]);
    }
  }
}

// Paired steps (several state groups, STATE_D >= 32).  There the fp32 MFMAs
// of the partials took half the kernel's time (the state groups' work-groups
// multiply the same history tiles, one per group), so a unit takes two
// history steps t0, t0+1 of its sample block and feeds
// v_mfma_f32_16x16x32_bf16 with K = 32 (sample, step) rows: row
// kappa = 8kg + 4s + i is sample 4kg+i at step t0+s, which is exactly what
// lane (kg, m) loads (A: its four rows at both steps; B: its d values at
// both steps).  fp32 history values and the d values are split exactly into
// three bf16 terms, and the six term products whose indices sum to at most
// 2 accumulate in fp32 (the three dropped ones are below 2^-23 of the
// product together, about one fp32 rounding); bf16 history values are
// exact, so three products.  The result layout is that of the fp32 MFMAs.
// Units per sample block: ceil(K/2) step pairs and the readout (its second
// half carries d = 0).  The second step of the last pair of an odd K
// re-reads step t0 with d masked to zero.  The history tiles are ordinary
// loads: the state
// groups' work-groups of a column block read them on one XCD and share them
// through L2.  32768 samples, K = 8, SH2 = 512, STATE_D = 64: 400-403 ->
// 333-337 us (327-334 us with the buffer loads below).  What remains is
// mostly VALU (the splits, the d values) and memory: with the MFMAs taken
// out the kernel still took 289 us where it took 351-361 us on the same
// machine.
struct BwdPair {
  v4f h[2][4];   // A operands: step s, row i (sample 4kg+i), 4 features
  v2u hr[2][4];  // bf16 inputs: the same, as loaded
  v4f al[2];     // alpha'_t of each step (readout: x_K)
  v4f be[2];     // beta'_t of each step
  v4f sr;        // S_r of the pair's round (both steps share it: rounds are 8 steps)
  float dc[4];   // d_context of samples 4kg+i, state n (0 for samples past B)
  int blk, tp, nvalid;  // block, pair (tp == ceil(K/2): readout), samples from the block's first to B
};

// Buffer loads with per-lane byte offsets fixed for the work-group: a unit
// changes only scalar descriptors (base and size), so its loads cost no
// VALU address arithmetic.  Each descriptor ends at the block's last sample
// below B, so rows past B read as zeros (history and d_context alike) and
// contribute nothing.  The offsets stay below 2^32 for K * SH2 <= 2^26.
struct PairLane {
  unsigned hs[4];  // history row 4kg+i of a block (step units), this lane's features
  unsigned ho[4];  // h_s2 row 4kg+i (readout units)
  unsigned dc[4];  // d_context row 4kg+i, this lane's state
  unsigned pl;     // this lane's float4 of a saved plane
};
template <class T>
__device__ __forceinline__ PairLane pair_lane(const BwdCtx<T>& c, int lane) {
  PairLane L;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned r = 4 * c.kg + i;
    L.hs[i] = (unsigned)(((size_t)r * c.K * c.SH2 + c.col) * sizeof(T));
    L.ho[i] = (unsigned)(((size_t)r * c.SH2 + c.col) * sizeof(T));
    L.dc[i] = (r * c.D + c.state) * sizeof(float);
  }
  L.pl = 16u * lane;
  return L;
}
__device__ __forceinline__ v4f ldb4(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <bool ROUNDS, class T>
__device__ __forceinline__ void bwd_load_pair(BwdPair& U, int u, const BwdCtx<T>& c, const PairLane& L) {
  const int ug = c.u0 + u;
  const int KP = c.UPB - 1;
  U.blk = ug / c.UPB;
  U.tp = ug - U.blk * c.UPB;
  U.nvalid = c.B - U.blk * kBlock;
  const int nv = min(U.nvalid, kBlock);
  const bool step = U.tp < KP;
  const int t0 = 2 * U.tp;
  // the pair's second step, when there is one (read as a scalar: the
  // descriptors below must stay in scalar registers)
  const int dt = __builtin_amdgcn_readfirstlane(step && t0 + 1 < c.K ? 1 : 0);
  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(c.saved + ((size_t)U.blk * c.NG + c.sg) * c.blk_stride, (unsigned)(c.blk_stride * sizeof(float)));
  constexpr unsigned PB = kPlane * sizeof(float);
  const unsigned p0 = step ? 2 * t0 : 2 * c.K;
  const unsigned p1 = step ? 2 * (t0 + dt) : 2 * c.K;
  U.al[0] = ldb4(rp, L.pl, p0 * PB);
  U.be[0] = ldb4(rp, L.pl, (step ? p0 + 1 : p0) * PB);
  U.al[1] = ldb4(rp, L.pl, p1 * PB);
  U.be[1] = ldb4(rp, L.pl, (step ? p1 + 1 : p1) * PB);
  if constexpr (ROUNDS) U.sr = ldb4(rp, L.pl, (step ? 2 * c.K + 1 + t0 / kChunk : 2 * c.K) * PB);
  // rows of the block at step t0 (or its h_s2 rows): the last valid row ends
  // after the pair's span
  const size_t rs = step ? (size_t)c.K * c.SH2 : (size_t)c.SH2;
  const T* base = step ? c.H + ((size_t)U.blk * kBlock * c.K + t0) * c.SH2 : c.hs2 + (size_t)U.blk * kBlock * c.SH2;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(base, (unsigned)(((size_t)(nv - 1) * rs + (size_t)(dt + 1) * c.SH2) * sizeof(T)));
  const unsigned s1 = (unsigned)(dt * c.SH2 * sizeof(T));
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(c.dctx + (size_t)U.blk * kBlock * c.D, (unsigned)(nv * c.D * sizeof(float)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned off = step ? L.hs[i] : L.ho[i];
    if constexpr (sizeof(T) == 2) {
      U.hr[0][i] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rh, off, 0, 0));
      U.hr[1][i] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rh, off, s1, 0));
    } else {
      U.h[0][i] = ldb4(rh, off, 0);
      U.h[1][i] = ldb4(rh, off, s1);
    }
    U.dc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, L.dc[i], 0, 0));
  }
}

template <bool DBG, bool ROUNDS, class T>
__device__ __forceinline__ void bwd_compute_pair(const BwdPair& U, bool live, const BwdCtx<T>& c, v4f (&acc)[4][3],
                                                 float* __restrict__ d_a_out, float* __restrict__ d_b_out,
                                                 float* __restrict__ d_c_out, bool write_dbg) {
  constexpr bool BF = sizeof(T) == 2;
  const int KP = c.UPB - 1;
  const bool step = U.tp < KP;
  const int t0 = 2 * U.tp;
  const bool two = step && t0 + 1 < c.K;
  const int sbase = U.blk * kBlock + 4 * c.kg;
  // d values, kappa order (4s + i); the readout's second half is zero
  float da[8], db[8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // rows past B arrive with d_context = 0
      const bool use = live && (s == 0 || two);
      const float dcs = use ? (ROUNDS && step ? U.dc[i] * U.sr[i] : U.dc[i]) : 0.f;
      da[4 * s + i] = dcs * U.al[s][i];
      db[4 * s + i] = dcs * U.be[s][i];
      if (DBG && write_dbg && use && 4 * c.kg + i < U.nvalid) {
        const int smp = sbase + i;
        if (step) {
          if (d_a_out) d_a_out[((size_t)smp * c.K + t0 + s) * c.D + c.state] = da[4 * s + i];
          if (d_b_out) d_b_out[((size_t)smp * c.K + t0 + s) * c.D + c.state] = db[4 * s + i];
        } else if (s == 0 && d_c_out) {
          d_c_out[(size_t)smp * c.D + c.state] = da[i];
        }
      }
    }
  // A operand of tile qq: feature 4m+qq at the eight (sample, step) rows
  auto hist = [&](int qq, v8bf (&xa)[BF ? 1 : 3]) {
    if constexpr (BF) {
      const int w = qq >> 1;
      const unsigned sel = (qq & 1) ? 0x07060302u : 0x05040100u;
      v4u p;
      p[0] = __builtin_amdgcn_perm(U.hr[0][1][w], U.hr[0][0][w], sel);
      p[1] = __builtin_amdgcn_perm(U.hr[0][3][w], U.hr[0][2][w], sel);
      p[2] = __builtin_amdgcn_perm(U.hr[1][1][w], U.hr[1][0][w], sel);
      p[3] = __builtin_amdgcn_perm(U.hr[1][3][w], U.hr[1][2][w], sel);
      xa[0] = __builtin_bit_cast(v8bf, p);
    } else {
      float x[8];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * s + i] = U.h[s][i][qq];
      split3_v8(x, xa);
    }
  };
  // term products (history term th, d term td) with th + td <= 2, the
  // smaller ones first; the step/readout choice is taken once per unit
  if (step) {
    v8bf ta[3], tb[3];
    split3_v8(da, ta);
    split3_v8(db, tb);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      v8bf xa[BF ? 1 : 3];
      hist(qq, xa);
#pragma unroll
      for (int td = 2; td >= 0; --td)
#pragma unroll
        for (int th = (BF ? 0 : 2 - td); th >= 0; --th) {
          acc[qq][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[th], ta[td], acc[qq][0], 0, 0, 0);
          acc[qq][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[th], tb[td], acc[qq][1], 0, 0, 0);
        }
    }
  } else {
    v8bf ta[3];
    split3_v8(da, ta);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      v8bf xa[BF ? 1 : 3];
      hist(qq, xa);
#pragma unroll
      for (int td = 2; td >= 0; --td)
#pragma unroll
        for (int th = (BF ? 0 : 2 - td); th >= 0; --th)
          acc[qq][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[th], ta[td], acc[qq][2], 0, 0, 0);
    }
  }
}

// Input gradients inside the backward (STATE_D = 16: the work-group's state
// group is every state).  A unit's d_h tile -- its 16 samples at this column
// block's 64 features -- is
//   d_h_history[b][t][j] = sum_s d_a[b,t,s] W_A[j][s] + d_b[b,t,s] W_B[j][s]
// (or d_h_s2[b][j] = sum_s d_c[b,s] W_C[j][s] for the readout), the chain
// rule through the projections.  The unit's d values go through the wave's
// LDS tile from the backward's layout (lane (kg, n): samples 4kg..4kg+3 of
// state n) to the B-operand layout of v_mfma_f32_16x16x32_bf16 (lane
// (kg, n): sample n, kappa = 8kg .. 8kg+7 of [d_a | d_b]), split exactly
// into three bf16 terms; W comes from LDS as three terms as well, and the
// six term products whose indices sum to at most 2 accumulate in fp32
// (M = 16 features x 4 tiles, N = the 16 samples, K = the 32 states).  The
// result agrees with mamba2_scan_bwd_input to fp32 rounding (that kernel
// uses fp32 MFMAs at STATE_D = 16).  Results leave through the same tile as
// 256-byte row pieces; a descriptor of the unit's valid rows drops the rest
// (and every store of a unit past the slice's last one).
constexpr int kFusedDRow = 20;             // padded row of the d transpose
// Row r of the d transpose: each 8-row group 16 floats further on, so that
// the column reads of lanes kg = 0, 1 (rows 8kg + e) fall in disjoint halves
// of the 32 banks; the 16-byte row writes of 8 lanes stay distinct.
__device__ __forceinline__ int fused_drow(int r) { return r * kFusedDRow + (r >> 3) * 16; }
constexpr int kFusedRow = kColBlock + 4;   // padded row of the output transpose
constexpr int kFusedTile = kBlock * kFusedRow;  // floats per wave (the d transpose takes fused_drow(31) + 20 = 688)
static_assert(31 * kFusedDRow + 3 * 16 + kFusedDRow <= kFusedTile, "the d transpose fits the tile");
// staged weights: per 16-feature tile jt, W_A|W_B (kappa = 0..31) and W_C
// (kappa = 0..15, zero above) as three bf16 terms in the
// v_mfma_f32_16x16x32_bf16 A-operand layout, [W_AB | W_C][jt][term][lane]
constexpr int kFusedW = 2 * 4 * 3 * 64 * 4;   // floats (16-byte entries)
__device__ __forceinline__ void din_fused(const float (&dv)[2][4], bool readout, bool live, int blk, int t,
                                          int B, int K, int SH2, int jb, int kg, int n, int lane,
                                          float* __restrict__ tile, const float* __restrict__ sW,
                                          float* __restrict__ dH, float* __restrict__ dhs2) {
  // (1) the transpose: row kappa = state (d_b 16 rows further), column = sample
  *reinterpret_cast<v4f*>(&tile[fused_drow(n) + 4 * kg]) = v4f{dv[0][0], dv[0][1], dv[0][2], dv[0][3]};
  *reinterpret_cast<v4f*>(&tile[fused_drow(kGroup + n) + 4 * kg]) = v4f{dv[1][0], dv[1][1], dv[1][2], dv[1][3]};
  __builtin_amdgcn_wave_barrier();
  // B operand, lane (kg, n): sample n at kappa = 8kg .. 8kg+7 (the readout:
  // d_c below 16, zero above), split exactly into three bf16 terms
  float d8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = tile[fused_drow(8 * kg + e) + n];
    d8[e] = (readout && kg >= 2) ? 0.f : x;
  }
  __builtin_amdgcn_wave_barrier();
  v8bf dt[3];
  split3_v8(d8, dt);
  // (2) per 16-feature tile jt: the six term products whose term indices
  // sum to at most 2 (the three dropped are below 2^-23 of the product
  // together), the result parked in the tile; (3) out through the tile:
  // lane (kg, n) then stores features 4n..4n+3 of samples 4i + kg
  const v4u* sw = reinterpret_cast<const v4u*>(sW) + (readout ? 4 * 3 * 64 : 0);
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tw = 2; tw >= 0; --tw) {
      const v8bf w = __builtin_bit_cast(v8bf, sw[(jt * 3 + tw) * 64 + lane]);
#pragma unroll
      for (int td = 2 - tw; td >= 0; --td) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, dt[td], acc, 0, 0, 0);
    }
    *reinterpret_cast<v4f*>(&tile[n * kFusedRow + jt * 16 + 4 * kg]) = acc;
  }
  __builtin_amdgcn_wave_barrier();
  const int nvalid = min(kBlock, B - blk * kBlock);
  float* out = readout ? dhs2 : dH;
  const size_t row_stride = readout ? (size_t)SH2 : (size_t)K * SH2;  // floats between samples
  float* base = out == nullptr ? nullptr
                               : out + (size_t)blk * kBlock * row_stride + (readout ? 0 : (size_t)t * SH2) +
                                     jb * kColBlock;
  const unsigned bytes = (out == nullptr || !live)
                             ? 0u
                             : (unsigned)(((size_t)(nvalid - 1) * row_stride + kColBlock) * sizeof(float));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4f v = *reinterpret_cast<const v4f*>(&tile[(4 * i + kg) * kFusedRow + 4 * n]);
    const unsigned off = (unsigned)(((size_t)(4 * i + kg) * row_stride + 4 * n) * sizeof(float));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), rs, off, 0, 0);
  }
  __builtin_amdgcn_wave_barrier();
}

// DIN (STATE_D = 16 only): also the input gradients d_h_history, d_h_s2 of
// each unit, from the same d values (see din_fused), with W_A, W_B, W_C of
// the column block staged in LDS.  The per-wave tiles and the staged W share
// the LDS of the final slice sum.
// NW waves per work-group: kBwdWaves, or 8 for the fp32 DIN form, which
// needs more than the 168 registers that three waves per SIMD leave.
template <class T, bool DBG, bool ROUNDS, bool DIN = false, int NW = kBwdWaves, bool PS = false>
__global__ __launch_bounds__(NW * 64) void bwd_partials_kernel(
    int B, int K, int SH2, int NG, int NB, int P, int UPW,
    const T* __restrict__ H, const T* __restrict__ hs2,
    const float* __restrict__ saved, const float* __restrict__ dctx,
    float* __restrict__ d_a_out, float* __restrict__ d_b_out, float* __restrict__ d_c_out,
    float* __restrict__ ws, const float* __restrict__ WA, const float* __restrict__ WB,
    const float* __restrict__ WC, float* __restrict__ dH, float* __restrict__ dhs2) {
  __shared__ __attribute__((aligned(16))) float sRed[NW][3 * kColBlock * kGroup];
  static_assert(NW * kFusedTile + kFusedW <= NW * 3 * kColBlock * kGroup, "fused tiles fit");

  const int NJB = SH2 / kColBlock;
  const int V = NJB * NG;
  const int xcd = blockIdx.x & 7;
  const int round = blockIdx.x >> 3;
  const int v = round % V;
  const int p = (round / V) * 8 + xcd;
  if (p >= P) return;
  const int jb = v % NJB;
  const int sg = v / NJB;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: unit indices stay scalar
  const int lane = tid & 63;
  const int kg = lane >> 4;
  const int m = lane & 15;
  const bool write_dbg = (jb == 0);

  BwdCtx<T> c;
  c.B = B;
  c.K = K;
  c.SH2 = SH2;
  c.D = NG * kGroup;
  c.NG = NG;
  c.sg = sg;
  c.u0 = p * UPW;
  c.col = jb * kColBlock + 4 * m;
  c.state = sg * kGroup + m;
  c.kg = kg;
  c.H = H;
  c.hs2 = hs2;
  c.saved = saved;
  c.dctx = dctx;
  c.blk_stride = (size_t)saved_planes(K) * kPlane;
  c.rounds = K > kChunk;
  c.hk_step = 4LL * kg * K * SH2;
  c.hk_out = 4LL * kg * SH2;
  c.UPB = PS ? (K + 1) / 2 + 1 : K + 1;
  const int n = min(NB * c.UPB - c.u0, UPW);

  v4f acc[4][3];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) acc[q][pl] = v4f{0.f, 0.f, 0.f, 0.f};

  constexpr int S = NW;
  if constexpr (PS) {
    // the same two-unit ring over step pairs
    BwdPair R0, R1;
    const PairLane L = pair_lane(c, lane);
    int u = wave;
    bwd_load_pair<ROUNDS>(R0, min(u, n - 1), c, L);
    for (; u < n; u += 2 * S) {
      bwd_load_pair<ROUNDS>(R1, min(u + S, n - 1), c, L);
      __builtin_amdgcn_sched_barrier(0);
      bwd_compute_pair<DBG, ROUNDS>(R0, u < n, c, acc, d_a_out, d_b_out, d_c_out, write_dbg);
      bwd_load_pair<ROUNDS>(R0, min(u + 2 * S, n - 1), c, L);
      __builtin_amdgcn_sched_barrier(0);
      bwd_compute_pair<DBG, ROUNDS>(R1, u + S < n, c, acc, d_a_out, d_b_out, d_c_out, write_dbg);
    }
  } else {
    // Two-unit ring.  Requests are unconditional: past the last unit a wave
    // re-loads the last unit (unused), so the compiler's waits stay exact.
    // Both halves of an iteration always run: a unit past the last one (u >= n)
    // re-reads and re-multiplies the last unit with its d_context masked to
    // zero, so the loop has no data-dependent exit between the two halves and
    // each unit's registers keep one role.
    BwdUnit R0, R1;
    int u = wave;
    bwd_load<ROUNDS>(R0, min(u, n - 1), c, lane);
    float* sW = &sRed[0][0] + NW * kFusedTile;         // DIN: staged weights
    float* tile = &sRed[0][0] + wave * kFusedTile;     // DIN: this wave's tile
    if constexpr (DIN) {
      // W of this column block as v_mfma_f32_16x16x32_bf16 A operands, three
      // exact bf16 terms each: entry (jt, lane (kg, m)) holds row jb*64 +
      // jt*16 + m at kappa = 8kg .. 8kg+7, W_A below 16 and W_B above for the
      // steps, W_C below 16 and zeros above for the readout
      for (int e = tid; e < 2 * 4 * 64; e += NW * 64) {
        const bool ro = e >= 4 * 64;
        const int l = e & 63, jt = (e >> 6) & 3, kgw = l >> 4;
        const float* row = (ro ? WC : (kgw < 2 ? WA : WB)) + (size_t)(jb * kColBlock + jt * 16 + (l & 15)) * kGroup +
                           8 * (kgw & 1);
        const v4f a = ld4(row), b = ld4(row + 4);
        const bool zero = ro && kgw >= 2;
        float v[8];
  #pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k] = zero ? 0.f : a[k];
          v[4 + k] = zero ? 0.f : b[k];
        }
        v8bf tw[3];
        split3_v8(v, tw);
        v4u* dst = reinterpret_cast<v4u*>(sW) + (ro ? 4 * 3 * 64 : 0);
  #pragma unroll
        for (int tm = 0; tm < 3; ++tm) dst[(jt * 3 + tm) * 64 + l] = __builtin_bit_cast(v4u, tw[tm]);
      }
      __syncthreads();
    }
    for (; u < n; u += 2 * S) {
      float dv[2][4];
      bwd_load<ROUNDS>(R1, min(u + S, n - 1), c, lane);
      __builtin_amdgcn_sched_barrier(0);
      bwd_compute<DBG, ROUNDS, sizeof(T) == 2>(R0, u < n, c, acc, d_a_out, d_b_out, d_c_out, write_dbg, dv);
      if constexpr (DIN) {
        din_fused(dv, R0.t == K, u < n, R0.blk, R0.t, B, K, SH2, jb, kg, m, lane, tile, sW, dH, dhs2);
        __builtin_amdgcn_sched_barrier(0);  // the next unit's loads stay after (registers)
      }
      bwd_load<ROUNDS>(R0, min(u + 2 * S, n - 1), c, lane);
      __builtin_amdgcn_sched_barrier(0);
      bwd_compute<DBG, ROUNDS, sizeof(T) == 2>(R1, u + S < n, c, acc, d_a_out, d_b_out, d_c_out, write_dbg, dv);
      if constexpr (DIN) {
        din_fused(dv, R1.t == K, u + S < n, R1.blk, R1.t, B, K, SH2, jb, kg, m, lane, tile, sW, dH, dhs2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // DIN: every wave is done with its tile and the staged W before sRed
  // (the same LDS) takes the partial sums
  if constexpr (DIN) __syncthreads();

  // Result lane (g = kg, n = m), element r of tile q: feature row
  // jl = 16*g + 4*r + q of the column block, state n.  Slices keep that
  // register order, [plane][g][q][n][r], so each lane writes whole float4s
  // (the reduce maps the order back onto dW).
#pragma unroll
  for (int pl = 0; pl < 3; ++pl)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<v4f*>(&sRed[wave][pl * (kColBlock * kGroup) + (kg * 4 + q) * 64 + m * 4]) = acc[q][pl];
  __syncthreads();

  // Slice layout: ws[sg][p][jb][plane][g][q][n][r].  Written through to memory
  // (16-byte stores with system-scope coherence) so that no dirty L2 lines
  // remain to be written back before the reduce can start.
  float* out = ws + ((size_t)sg * P + p) * ((size_t)SH2 * 3 * kGroup) + (size_t)jb * (3 * kColBlock * kGroup);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(out, 3 * kColBlock * kGroup * sizeof(float));
  for (int e = 4 * tid; e < 3 * kColBlock * kGroup; e += 4 * NW * 64) {
    v4f s = *reinterpret_cast<const v4f*>(&sRed[0][e]);
#pragma unroll
    for (int w = 1; w < NW; ++w) s += *reinterpret_cast<const v4f*>(&sRed[w][e]);
    st4_through(rs, (unsigned)(e * sizeof(float)), s);
  }
}

// ---------------------------------------------------------------------------
// Backward, phase 2: dW = sum over slices p = 0..P-1, in a fixed order.
//   grid = ceil(NG * SH2 * 48 / 4 / 32), 256 threads: 32 element quads x 8
//   contiguous slice groups; the groups are combined in order 0..7.
// Fixed-order sum of P slices (stride `stride` floats) of one float4 per
// thread group: 8 contiguous groups of slices, then the groups in order.
__device__ __forceinline__ v4f reduce_slices(const float* __restrict__ src, size_t stride, int P, bool ok, int grp,
                                             int ql, v4f (*sPart)[kRedQuads]) {
  const int pc = (P + kRedGroups - 1) / kRedGroups;
  const int p0 = grp * pc;
  const int p1 = min(P, p0 + pc);
  v4f s = {0.f, 0.f, 0.f, 0.f};
  // Eight loads in flight per pass, all unconditional (clamped to a valid
  // slice); a load past the group's slices, or of a thread with no output,
  // is not added.  The sum runs over p0 .. p1-1 in order.
  for (int b = p0; b < p0 + pc; b += 8) {
    v4f v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ld4(src + (size_t)min(b + j, P - 1) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const v4f t = s + v[j];
      s = (ok && b + j < p1) ? t : s;
    }
  }
  sPart[grp][ql] = s;
  __syncthreads();
  v4f tot = sPart[0][ql];
#pragma unroll
  for (int g = 1; g < kRedGroups; ++g) tot += sPart[g][ql];
  return tot;
}

// The dW blocks come first; when dw is given, SH2/128 more blocks sum the
// blend's d_temporal_weight slices (Pw of SH2 floats at wsw) and scale by 1/D.
__global__ __launch_bounds__(kRedThreads) void bwd_reduce_kernel(
    int SH2, int NG, int P, const float* __restrict__ ws,
    float* __restrict__ dWA, float* __restrict__ dWB, float* __restrict__ dWC,
    int Pw, const float* __restrict__ wsw, float* __restrict__ dw) {
  __shared__ v4f sPart[kRedGroups][kRedQuads];
  const int per_sg = SH2 * 3 * kGroup;
  const int quads = NG * per_sg / 4;
  const int dw_blocks = (quads + kRedQuads - 1) / kRedQuads;
  const int ql = threadIdx.x % kRedQuads;
  const int grp = threadIdx.x / kRedQuads;
  const int D = NG * kGroup;

  if ((int)blockIdx.x >= dw_blocks) {
    const int qd = ((int)blockIdx.x - dw_blocks) * kRedQuads + ql;
    const bool ok = qd < SH2 / 4;
    const v4f tot = reduce_slices(wsw + (ok ? 4 * qd : 0), (size_t)SH2, Pw, ok, grp, ql, sPart);
    if (grp != 0 || !ok) return;
    const float inv = 1.f / (float)D;
#pragma unroll
    for (int r = 0; r < 4; ++r) dw[4 * qd + r] = tot[r] * inv;
    return;
  }

  const int qd = blockIdx.x * kRedQuads + ql;
  const bool ok = qd < quads;
  const int e = ok ? qd * 4 : 0;
  const int sg = e / per_sg;
  const int o = e - sg * per_sg;
  const v4f tot = reduce_slices(ws + (size_t)sg * P * per_sg + o, (size_t)per_sg, P, ok, grp, ql, sPart);
  if (grp != 0 || !ok) return;

  // slice order [jb][plane][g][q][n][r]: element r of this quad is feature
  // row jl = 16g + 4r + q of column block jb, state n
  const int jb = o / (3 * kColBlock * kGroup);
  const int rem = o - jb * (3 * kColBlock * kGroup);
  const int pl = rem / (kColBlock * kGroup);
  const int rem2 = rem - pl * (kColBlock * kGroup);
  const int g = rem2 >> 8, q = (rem2 >> 6) & 3, n = (rem2 >> 2) & 15;
  float* dst = (pl == 0 ? dWA : (pl == 1 ? dWB : dWC)) + (size_t)(jb * kColBlock + 16 * g + q) * D + sg * kGroup + n;
#pragma unroll
  for (int r = 0; r < 4; ++r) dst[(size_t)(4 * r) * D] = tot[r];
}

// ---------------------------------------------------------------------------
// The h_enriched blend, the step after the path (implementation plan, Task 1
// step 3): h_enriched[b][j] = h_s2[b][j] + w_j * (sum_s context[b][s]) / D
// with w = temporal_weight (1 for every feature when absent).  Its backward,
// by the chain rule: dL/d(sum_s context[b][s]) = (d_h_enriched[b,:] . w) / D
// is every state's d_context, and d_temporal_weight[j] =
// sum_b d_h_enriched[b][j] (sum_s context[b][s]) / D.  One wave per sample
// row; a lane holds features 4l..4l+3 (and 256 + 4l.. when SH2 > 256).
constexpr int kBlendWaves = 8;
constexpr int kBlendSlices = 256;  // most d_temporal_weight slices (one per backward work-group)

__device__ __forceinline__ float wave_sum(float v) {
  // butterfly over the 64 lanes: the same fixed order on every call
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(kBlendWaves * 64) void blend_fwd_kernel(
    int B, int SH2, int D, const float* __restrict__ ctx, const float* __restrict__ hs2,
    const float* __restrict__ w, float* __restrict__ he) {
  const int b = blockIdx.x * kBlendWaves + (threadIdx.x >> 6);
  if (b >= B) return;
  const int lane = threadIdx.x & 63;
  float sum = 0.f;
  for (int s = 0; s < D; ++s) sum += ctx[(size_t)b * D + s];  // states in order
  const float scale = sum * (1.f / (float)D);                  // exact: D is a power of two
  for (int j = 4 * lane; j < SH2; j += 256) {
    const v4f h = ld4(hs2 + (size_t)b * SH2 + j);
    const v4f wv = w != nullptr ? ld4(w + j) : v4f{1.f, 1.f, 1.f, 1.f};
    v4f o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = h[r] + wv[r] * scale;
    *reinterpret_cast<v4f*>(he + (size_t)b * SH2 + j) = o;
  }
}

//   grid = ceil(B / RPW), 512 threads: work-group p takes samples
//   [p*RPW, (p+1)*RPW), wave w every 8th of them; it writes every state's
//   d_context of its samples and slice p of d_temporal_weight (before the
//   1/D), the waves' partials summed in wave order.  sum_s context[b][s] is
//   rebuilt from the saved planes: c = beta'_{K-1} (no later gate) and x_K.
__global__ __launch_bounds__(kBlendWaves * 64) void blend_bwd_kernel(
    int B, int K, int SH2, int NG, int RPW, const float* __restrict__ saved, const float* __restrict__ w,
    const float* __restrict__ dhe, float* __restrict__ dctx, float* __restrict__ wpart) {
  __shared__ v4f sPart[kBlendWaves][128];  // SH2 / 4 <= 128
  const int p = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int D = NG * kGroup;
  const size_t blk_stride = (size_t)saved_planes(K) * kPlane;
  v4f wv[2], acc[2];
  bool act[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int col = 4 * lane + 256 * r;
    act[r] = col < SH2;
    wv[r] = (act[r] && w != nullptr) ? ld4(w + col) : v4f{1.f, 1.f, 1.f, 1.f};
    acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const int b0 = p * RPW;
  const int b1 = min(B, b0 + RPW);
  // A wave's rows come kBlendRows at a time, every load of the batch issued
  // before the first is used (a row's own work is two wave sums); a row past
  // the slice re-loads the slice's last row and contributes nothing.
  constexpr int kBlendRows = 4;
  const int ls = min(lane, D - 1);  // state of this lane's saved-plane loads
  for (int bb = b0 + wave; bb < b1; bb += kBlendWaves * kBlendRows) {
    v4f dv[kBlendRows][2];
    float cb[kBlendRows], cxk[kBlendRows];
#pragma unroll
    for (int i = 0; i < kBlendRows; ++i) {
      const int b = min(bb + i * kBlendWaves, b1 - 1);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        dv[i][r] = ld4(dhe + (size_t)b * SH2 + min(4 * lane + 256 * r, SH2 - 4));
      const float* sv = saved + ((size_t)(b >> 4) * NG + (ls >> 4)) * blk_stride;
      const int pi = plane_index(b & 15, ls & 15);
      cb[i] = sv[(size_t)(2 * K - 1) * kPlane + pi];
      cxk[i] = sv[(size_t)(2 * K) * kPlane + pi];
    }
#pragma unroll
    for (int i = 0; i < kBlendRows; ++i) {
      const int b = bb + i * kBlendWaves;
      const bool live = b < b1;
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) part += act[r] ? dv[i][r][q] * wv[r][q] : 0.f;
      const float dsum = wave_sum(part) * (1.f / (float)D);
      if (live && lane < D) dctx[(size_t)b * D + lane] = dsum;
      const float csum = wave_sum(lane < D ? cb[i] * cxk[i] : 0.f);
#pragma unroll
      for (int r = 0; r < 2; ++r) acc[r] += live && act[r] ? dv[i][r] * csum : v4f{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (act[r]) sPart[wave][lane + 64 * r] = acc[r];
  __syncthreads();
  for (int e = threadIdx.x; e < SH2 / 4; e += kBlendWaves * 64) {
    v4f t = sPart[0][e];
#pragma unroll
    for (int v = 1; v < kBlendWaves; ++v) t += sPart[v][e];
    *reinterpret_cast<v4f*>(wpart + (size_t)p * SH2 + 4 * e) = t;
  }
}

// ---------------------------------------------------------------------------
// Input gradients, an optional step past the pages' path (their backward
// ends with the weight gradients).  By the chain rule through the three
// projections:
//   d_h_history[b][t][j] = sum_s d_a[b,t,s] W_A[j][s] + d_b[b,t,s] W_B[j][s]
//   d_h_s2[b][j]         = sum_s d_c[b,s]   W_C[j][s]
// with d_a, d_b, d_c formed from `saved` and d_context exactly as in the
// backward.  Neither h_history nor h_s2 is read.
//   grid = 8 * (SH2/64) * ceil(NSL / 8), 256 threads.  A unit is (sample
//   block, step t) for t < K, or the readout (t = K), numbered block-major;
//   work-group: a slice of UPW consecutive units (so few samples with a long
//   history still spread over ~1024 work-groups, up to kDinMaxWGs with one
//   state group) and one 64-feature column
//   block; the column blocks of a slice run on one XCD so they share the
//   saved planes in L2.  Wave w takes units w, w+4, ... of its slice.  With
//   one state group it loads all of them (up to kDinBatch) before its first
//   store; otherwise it requests the next unit's operands while it
//   multiplies the current one.
// Operands: a unit's saved planes and the block's d_context arrive as whole
// 1 KiB rows (one 16-byte load per lane each, four per unit at D = 16) and
// pass through the wave's LDS tile into the MFMA layout.  The kernel writes
// eight times what it reads, so every load waits behind queued stores in
// the CU's memory pipeline; few, wide loads keep that pipeline short.
// MFMA roles: M = 16 features (4 tiles), N = the 16 samples, K = the 2*D
// (or D) states, in the order described at DinW; B lane (kg, n) holds
// d[sample n][the same state] from the tile.  Results leave
// through the wave's LDS tile as 256-byte row pieces (stores in 64-byte
// pieces fall well short of the HBM write rate).
// Every unit issues the same loads (a readout loads x_K where a step loads
// alpha' and beta') and the same four stores, range-checked by a buffer
// descriptor rather than by a branch, so the compiler's memory-counter waits
// stay exact and the next unit's requests stay in flight.
constexpr int kDinWaves = 4;
// One state group: each wave issues the loads of all its units (at most
// kDinBatch) before its first store.  A CU's memory pipe completes requests
// in issue order, so a unit's loads issued after earlier units' stores waited
// for those stores (4 KiB per unit) to drain; loaded up front, a unit's data
// is there when the wave reaches it (24.5 -> 21.2 us at 8192 samples).
constexpr int kDinBatch = 6;
constexpr long long kDinMaxWGs = 4096;  // one state group: a longer slice beyond this many work-groups
constexpr int kDinTargetWGs = 4096 / kDinWaves;      // 16 resident waves per CU
constexpr int kDinTargetWGsRounds = 2 * kDinTargetWGs;  // multi-round histories: shorter slices balance better
constexpr int kDinRow = kColBlock + 4;               // padded LDS row of the output transpose
constexpr int kDinPlaneLds = kPlane + 16;            // padded LDS copy of a saved plane
// A saved plane in LDS: its four sample quads 68 floats apart instead of 64,
// so that the B-operand reads (lane (kg, n): sample n, states 4kg + c) of one
// q-step touch 64 different banks.
__device__ __forceinline__ int din_pad(int e) { return e + (e >> 6) * 4; }
constexpr long long kDinMaxRowFloats = 1LL << 26;    // K * SH2 limit: 16 rows of samples stay below 4 GiB

// LDS floats of one wave's tile: the unit's planes (alpha', beta', S_r; NGT
// of each) and the block's d_context rows (padded by 4 floats), reused
// afterwards for the output transpose.
__host__ __device__ constexpr int din_tile_floats(int ngt) {
  return 3 * ngt * kDinPlaneLds + kBlock * (ngt * kGroup + 4) > kBlock * kDinRow
             ? 3 * ngt * kDinPlaneLds + kBlock * (ngt * kGroup + 4)
             : kBlock * kDinRow;
}

template <int NGT>
struct DinUnit {
  v4f pa[NGT];  // alpha'_t (step) or x_K (readout) plane of each state group
  v4f pb[NGT];  // beta'_t (step) or x_K again (readout)
  v4f ps[NGT];  // S_r plane of the step's round (multi-round histories only)
  v4f pd[NGT];  // the block's d_context rows, sample-major
};

struct DinCtx {
  int B, K, u0;  // u0: the work-group's first unit (units are (block, t), t-minor)
  size_t blk_stride;
  const float* saved;
  const float* dctx;
};

template <int NGT, bool ROUNDS>
__device__ __forceinline__ void din_load(DinUnit<NGT>& U, int u, const DinCtx& c, int lane) {
  constexpr int D = NGT * kGroup;
  const int KU = c.K + 1;
  const int blk = (c.u0 + u) / KU;
  const int t = c.u0 + u - blk * KU;
  const bool step = t < c.K;
  const int p0 = step ? 2 * t : 2 * c.K;
  const int p1 = step ? 2 * t + 1 : 2 * c.K;
  const int ps = 2 * c.K + 1 + (step ? t / kChunk : 0);
  const float* sv = c.saved + (size_t)blk * NGT * c.blk_stride + 4 * lane;
  // d_context rows of the block; rows past B are clamped to row B-1 (their
  // results are never stored)
  const int nrow = c.B - blk * kBlock;
  const float* dc = c.dctx + (size_t)blk * kBlock * D;
#pragma unroll
  for (int g = 0; g < NGT; ++g) {
    const float* gp = sv + (size_t)g * c.blk_stride;
    U.pa[g] = ld4(gp + (size_t)p0 * kPlane);
    U.pb[g] = ld4(gp + (size_t)p1 * kPlane);
    if (ROUNDS) U.ps[g] = ld4(gp + (size_t)ps * kPlane);
    const int e = (g * 64 + lane) * 4;  // float index in the block's [16][D] rows
    const int row = min(e / D, nrow - 1);
    U.pd[g] = ld4(dc + (size_t)row * D + (e % D));
  }
}

// The column block's weights as MFMA A operands.  Contraction element of
// q-step q for lane kg: kappa = 16*(q/4) + 4*kg + q%4 (kappa < D: state kappa
// of W_A; kappa >= D: state kappa - D of W_B), so the four q-steps 4qq..4qq+3
// of lane (kg, m) are one contiguous float4 of a W row, staged in the
// work-group's LDS.  (Holding them in registers instead, at D = 16, was no
// faster.)
__device__ __forceinline__ const float* din_w_src(const float* WA, const float* WB, int NGT, int qq) {
  return qq < NGT ? WA : WB;
}

template <int NGT>
struct DinW {
  static constexpr bool kSplit = false;
  const float* sab;  // [jt][qq][lane] float4
  const float* sc;
  int lane;
  __device__ __forceinline__ v4f AB(int jt, int qq) const {
    return *reinterpret_cast<const v4f*>(&sab[((jt * 2 * NGT + qq) * 64 + lane) * 4]);
  }
  __device__ __forceinline__ v4f C(int jt, int qq) const {
    return *reinterpret_cast<const v4f*>(&sc[((jt * NGT + qq) * 64 + lane) * 4]);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t din_rsrc(float* base, unsigned bytes) { return make_rsrc(base, bytes); }

// Split weights (D >= 32): the contraction runs on v_mfma_f32_16x16x32_bf16, K
// chunk h covering kappa = 32h + 8kg + e (e = 0..7) for lane kg, with
// kappa < D state kappa of W_A / d_a and kappa >= D state kappa - D of
// W_B / d_b (the readout: W_C / d_c, zero past D).  Weights and d are split
// exactly into three bf16 terms each and the six products with term
// indices summing to at most 2 accumulate in fp32 (the dropped three are
// below 2^-23 of the product together).
template <int NGT>
struct DinWs {
  static constexpr bool kSplit = true;
  static constexpr int NCS = NGT;                         // K chunks of a step unit (2D / 32)
  static constexpr int NCR = (NGT * kGroup + 31) / 32;    // K chunks of a readout unit
  // readout lanes kept: at D = 16 the lanes kg = 2, 3 of its one chunk
  // carry kappa >= D, all zero, and are not stored
  static constexpr int RL = NGT == 1 ? 32 : 64;
  const v4u* ss;  // [jt][h][term][lane]
  const v4u* sr;  // [jt][h][term][lane < RL]
  int lane;
  __device__ __forceinline__ v8bf S(int jt, int h, int tm) const {
    return __builtin_bit_cast(v8bf, ss[((jt * NCS + h) * 3 + tm) * 64 + lane]);
  }
  __device__ __forceinline__ v8bf R(int jt, int h, int tm) const {
    const v4u w = lane < RL ? sr[((jt * NCR + h) * 3 + tm) * RL + lane] : v4u{0u, 0u, 0u, 0u};
    return __builtin_bit_cast(v8bf, w);
  }
};


template <int NGT, bool ROUNDS, class WOps>
__device__ __forceinline__ void din_compute(const DinUnit<NGT>& U, int u, const DinCtx& c, int SH2, int jb, int kg,
                                            int n, const WOps& W, float* __restrict__ tile, int lane,
                                            float* __restrict__ dH, float* __restrict__ dhs2) {
  constexpr int D = NGT * kGroup;
  constexpr int NQ = D / 4;
  const int KU = c.K + 1;
  const int blk = (c.u0 + u) / KU;
  const int t = c.u0 + u - blk * KU;
  const bool readout = t == c.K;

  // operands into the tile: [kind][group] planes, then the d_context rows
  float* tA = tile;
  float* tB = tile + NGT * kDinPlaneLds;
  float* tS = tile + 2 * NGT * kDinPlaneLds;
  float* tD = tile + 3 * NGT * kDinPlaneLds;
#pragma unroll
  for (int g = 0; g < NGT; ++g) {
    *reinterpret_cast<v4f*>(&tA[g * kDinPlaneLds + din_pad(4 * lane)]) = U.pa[g];
    *reinterpret_cast<v4f*>(&tB[g * kDinPlaneLds + din_pad(4 * lane)]) = U.pb[g];
    if (ROUNDS) *reinterpret_cast<v4f*>(&tS[g * kDinPlaneLds + din_pad(4 * lane)]) = U.ps[g];
    {
      // d_context rows 4 floats apart beyond their D (fewer bank conflicts
      // in the column reads below)
      const int e = (g * 64 + lane) * 4;
      *reinterpret_cast<v4f*>(&tD[(e / D) * (D + 4) + e % D]) = U.pd[g];
    }
  }
  __builtin_amdgcn_wave_barrier();
  v4f acc[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) acc[jt] = v4f{0.f, 0.f, 0.f, 0.f};
  if constexpr (WOps::kSplit) {
    // lane (kg, n): the eight d values of its K-chunk slots, sample n
    constexpr int NCH = WOps::NCS;  // at least NCR
    const int nch = readout ? WOps::NCR : WOps::NCS;
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
      if (h >= nch) break;  // uniform: the unit's kind
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kap = 32 * h + 8 * kg + e;
        const int st = kap < D ? kap : kap - D;  // state
        const int pidx = (st >> 4) * kDinPlaneLds + din_pad(plane_index(n, st & 15));
        float dc = tD[n * (D + 4) + st];
        if (ROUNDS && !readout) dc *= tS[pidx];
        const float x = (readout || kap < D) ? tA[pidx] : tB[pidx];
        v[e] = (readout && kap >= D) ? 0.f : dc * x;
      }
      v8bf dt[3];
      split3_v8(v, dt);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int tw = 2; tw >= 0; --tw) {
          const v8bf w = readout ? W.R(jt, h, tw) : W.S(jt, h, tw);
#pragma unroll
          for (int td = 2 - tw; td >= 0; --td)
            acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, dt[td], acc[jt], 0, 0, 0);
        }
    }
    __builtin_amdgcn_wave_barrier();
  } else {
  // B operands: lane (kg, n) at q-step i holds state 16(i/4) + 4kg + i%4 of
  // sample n (d_a for q-step i, d_b for q-step i + NQ)
  float da[NQ], db[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int sn = 4 * kg + (i & 3);
    const int pidx = (i >> 2) * kDinPlaneLds + din_pad(plane_index(n, sn));
    float dc = tD[n * (D + 4) + 16 * (i >> 2) + sn];
    if (ROUNDS && !readout) dc *= tS[pidx];
    da[i] = dc * tA[pidx];
    db[i] = dc * tB[pidx];
  }
  __builtin_amdgcn_wave_barrier();

  if (!readout) {
    // q-steps 0..NQ-1 contract d_a with W_A, NQ..2NQ-1 d_b with W_B
#pragma unroll
    for (int qq = 0; qq < 2 * NQ / 4; ++qq) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const v4f w = W.AB(jt, qq);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = 4 * qq + i;
          acc[jt] = mfma16x16x4(w[i], q < NQ ? da[q] : db[q - NQ], acc[jt]);
        }
      }
    }
  } else {
    // readout: da holds d_c = d_context * x_K
#pragma unroll
    for (int qq = 0; qq < NQ / 4; ++qq) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const v4f w = W.C(jt, qq);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[jt] = mfma16x16x4(w[i], da[4 * qq + i], acc[jt]);
      }
    }
  }
  }
  // Result lane (kg, n), element r: feature jt*16 + 4kg + r of the column
  // block, sample n.  Transposed through the tile so that lane (kg, n) then
  // stores features 4n..4n+3 of samples 4i+kg, i = 0..3.
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) *reinterpret_cast<v4f*>(&tile[n * kDinRow + jt * 16 + 4 * kg]) = acc[jt];
  __builtin_amdgcn_wave_barrier();
  // Descriptor based at (first sample of the block, this unit's row, column
  // block); its size ends after the last valid sample's 64 features, so the
  // rows of samples >= B (and every store, for an output not requested) are
  // dropped by the range check.
  const int nvalid = min(kBlock, c.B - blk * kBlock);
  float* out = readout ? dhs2 : dH;
  const size_t row_stride = readout ? (size_t)SH2 : (size_t)c.K * SH2;  // floats between samples
  float* base = out == nullptr ? nullptr
                               : out + (size_t)blk * kBlock * row_stride + (readout ? 0 : (size_t)t * SH2) +
                                     jb * kColBlock;
  const unsigned bytes =
      out == nullptr ? 0u : (unsigned)(((size_t)(nvalid - 1) * row_stride + kColBlock) * sizeof(float));
  const __amdgpu_buffer_rsrc_t rs = din_rsrc(base, bytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4f v = *reinterpret_cast<const v4f*>(&tile[(4 * i + kg) * kDinRow + 4 * n]);
    const unsigned off = (unsigned)(((size_t)(4 * i + kg) * row_stride + 4 * n) * sizeof(float));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), rs, off, 0, 0);
  }
  __builtin_amdgcn_wave_barrier();
}

template <int NGT, bool ROUNDS>
__global__ __launch_bounds__(kDinWaves * 64) void dinput_kernel(
    int B, int K, int SH2, int NB, int UPW,
    const float* __restrict__ WA, const float* __restrict__ WB, const float* __restrict__ WC,
    const float* __restrict__ saved, const float* __restrict__ dctx,
    float* __restrict__ dH, float* __restrict__ dhs2) {
  constexpr int D = NGT * kGroup;
  // weights: [tile jt][q-step group qq][lane] float4, or (split) three bf16
  // terms per [tile jt][K chunk h][lane]
  // split weights pay from two state groups on (at D = 16 the per-unit
  // split of d and the larger weight tile cost more than the MFMAs saved)
  constexpr bool SPLIT = NGT >= 2;
  using WS = DinWs<NGT>;
  __shared__ float sWab[SPLIT ? 4 : 4 * 2 * NGT * 64 * 4];
  __shared__ float sWc[SPLIT ? 4 : 4 * NGT * 64 * 4];
  __shared__ v4u sWs[SPLIT ? 4 * WS::NCS * 3 * 64 : 1];
  __shared__ v4u sWr[SPLIT ? 4 * WS::NCR * 3 * WS::RL : 1];
  __shared__ float sTile[kDinWaves][din_tile_floats(NGT)];

  const int NJB = SH2 / kColBlock;
  const int xcd = blockIdx.x & 7;
  const int round = blockIdx.x >> 3;
  const int jb = round % NJB;
  const int slice = (round / NJB) * 8 + xcd;
  const int total = NB * (K + 1);
  DinCtx c;
  c.u0 = slice * UPW;
  if (c.u0 >= total) return;
  c.B = B;
  c.K = K;
  c.blk_stride = (size_t)saved_planes(K) * kPlane;
  c.saved = saved;
  c.dctx = dctx;
  const int n_units = min(UPW, total - c.u0);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int kg = lane >> 4;
  const int n = lane & 15;

  constexpr int S = kDinWaves;
  constexpr bool BATCH = NGT == 1;  // every unit loaded up front (UPW <= kDinBatch * S)
  DinUnit<NGT> R0, R1;
  DinUnit<NGT> UB[BATCH ? kDinBatch : 1];
  // The ring: the first unit's operands go out before the weights.
  if constexpr (!BATCH) din_load<NGT, ROUNDS>(R0, min(wave, n_units - 1), c, lane);

  if constexpr (SPLIT) {
    // lane l of (tile jt, chunk h): feature row jb*64 + jt*16 + l%16, the
    // eight weights of kappa = 32h + 8(l/16) .. +7 (W_A below D, W_B above;
    // W_C below D and zeros above for the readout), three terms each
    for (int e = tid; e < 4 * WS::NCS * 64 + 4 * WS::NCR * WS::RL; e += kDinWaves * 64) {
      const bool ro = e >= 4 * WS::NCS * 64;
      const int ee = ro ? e - 4 * WS::NCS * 64 : e;
      const int nc = ro ? WS::NCR : WS::NCS;
      const int nl = ro ? WS::RL : 64;
      const int l = ee % nl, h = (ee / nl) % nc, jt = (ee / nl) / nc;
      const size_t row = (size_t)(jb * kColBlock + jt * 16 + (l & 15)) * D;
      const int k0 = 32 * h + 8 * (l >> 4);
      float v[8];
      if (ro && k0 >= D) {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      } else {
        const float* src = ro ? WC + row + k0 : (k0 < D ? WA + row + k0 : WB + row + (k0 - D));
        const v4f a = ld4(src), b = ld4(src + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k] = a[k];
          v[4 + k] = b[k];
        }
      }
      v8bf tw[3];
      split3_v8(v, tw);
      v4u* dst = ro ? sWr : sWs;
#pragma unroll
      for (int tm = 0; tm < 3; ++tm) dst[((jt * nc + h) * 3 + tm) * nl + l] = __builtin_bit_cast(v4u, tw[tm]);
    }
  } else if constexpr (BATCH) {
    // The weights' loads go out first (they return first), then every
    // unit's (a slot past the last unit re-loads it, unused), then the
    // weights go into LDS.
    static_assert(4 * 2 * NGT * 64 == 2 * kDinWaves * 64 && 4 * NGT * 64 == kDinWaves * 64, "one W_C, two W_A|W_B float4s per thread");
    v4f wab[2], wcv;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + i * kDinWaves * 64;
      const int l = e & 63, qq = (e >> 6) % (2 * NGT), jt = (e >> 6) / (2 * NGT);
      const size_t row = (size_t)(jb * kColBlock + jt * 16 + (l & 15)) * D + 4 * (l >> 4);
      wab[i] = ld4(din_w_src(WA, WB, NGT, qq) + row + 16 * (qq % NGT));
    }
    {
      const int l = tid & 63, jt = tid >> 6;
      const size_t row = (size_t)(jb * kColBlock + jt * 16 + (l & 15)) * D + 4 * (l >> 4);
      wcv = ld4(WC + row);
    }
#pragma unroll
    for (int k = 0; k < kDinBatch; ++k) din_load<NGT, ROUNDS>(UB[k], min(wave + k * S, n_units - 1), c, lane);
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<v4f*>(&sWab[(tid + i * kDinWaves * 64) * 4]) = wab[i];
    *reinterpret_cast<v4f*>(&sWc[tid * 4]) = wcv;
  } else {
    for (int e = tid; e < 4 * 2 * NGT * 64; e += kDinWaves * 64) {
      const int l = e & 63, qq = (e >> 6) % (2 * NGT), jt = (e >> 6) / (2 * NGT);
      const size_t row = (size_t)(jb * kColBlock + jt * 16 + (l & 15)) * D + 4 * (l >> 4);
      *reinterpret_cast<v4f*>(&sWab[e * 4]) = ld4(din_w_src(WA, WB, NGT, qq) + row + 16 * (qq % NGT));
    }
    for (int e = tid; e < 4 * NGT * 64; e += kDinWaves * 64) {
      const int l = e & 63, qq = (e >> 6) % NGT, jt = (e >> 6) / NGT;
      const size_t row = (size_t)(jb * kColBlock + jt * 16 + (l & 15)) * D + 4 * (l >> 4);
      *reinterpret_cast<v4f*>(&sWc[e * 4]) = ld4(WC + row + 16 * qq);
    }
  }
  std::conditional_t<SPLIT, DinWs<NGT>, DinW<NGT>> W;
  if constexpr (SPLIT) {
    W.ss = sWs;
    W.sr = sWr;
  } else {
    W.sab = sWab;
    W.sc = sWc;
  }
  W.lane = lane;
  __syncthreads();

  if constexpr (BATCH) {
#pragma unroll
    for (int k = 0; k < kDinBatch; ++k) {
      const int u = wave + k * S;
      if (u < n_units) din_compute<NGT, ROUNDS>(UB[k], u, c, SH2, jb, kg, n, W, sTile[wave], lane, dH, dhs2);
    }
    // further batches: slices longer than one batch per wave (large inputs,
    // whose grid is held to kDinMaxWGs)
    for (int b0 = wave + kDinBatch * S; b0 < n_units; b0 += kDinBatch * S) {
#pragma unroll
      for (int k = 0; k < kDinBatch; ++k) din_load<NGT, ROUNDS>(UB[k], min(b0 + k * S, n_units - 1), c, lane);
#pragma unroll
      for (int k = 0; k < kDinBatch; ++k) {
        const int u = b0 + k * S;
        if (u < n_units) din_compute<NGT, ROUNDS>(UB[k], u, c, SH2, jb, kg, n, W, sTile[wave], lane, dH, dhs2);
      }
    }
    return;
  }
  // Two-unit ring; a request past the last unit re-loads the last unit (unused).
  for (int u = wave; u < n_units; u += 2 * S) {
    din_load<NGT, ROUNDS>(R1, min(u + S, n_units - 1), c, lane);
    __builtin_amdgcn_sched_barrier(0);
    din_compute<NGT, ROUNDS>(R0, u, c, SH2, jb, kg, n, W, sTile[wave], lane, dH, dhs2);
    if (u + S >= n_units) break;
    din_load<NGT, ROUNDS>(R0, min(u + 2 * S, n_units - 1), c, lane);
    __builtin_amdgcn_sched_barrier(0);
    din_compute<NGT, ROUNDS>(R1, u + S, c, SH2, jb, kg, n, W, sTile[wave], lane, dH, dhs2);
  }
}

// ---------------------------------------------------------------------------
// Host side: shape checks and launch plans.
struct Plan {
  int B, K, SH2, D, NG, NB, NJB, V;
  int P, UPW;  // backward slices and units per slice
  size_t saved_bytes, ws_bytes;
};

int make_plan(int B, int K, int SH2, int D, Plan* pl) {
  if (B <= 0 || K <= 0 || SH2 <= 0 || D <= 0) return MAMBA2_SCAN_EBADDIM;
  if (D != 16 && D != 32 && D != 64) return MAMBA2_SCAN_EUNSUPPORTED;
  if (SH2 % kColBlock != 0 || SH2 > 512) return MAMBA2_SCAN_EUNSUPPORTED;
  // Every element offset must fit comfortably in 64 bits and every block and
  // unit count in 32 bits.
  const long long rows = (long long)B * K;
  if (rows > (1LL << 40) / SH2) return MAMBA2_SCAN_EBADDIM;
  pl->B = B;
  pl->K = K;
  pl->SH2 = SH2;
  pl->D = D;
  pl->NG = D / kGroup;
  pl->NB = (B + kBlock - 1) / kBlock;
  if ((long long)pl->NB * K > (1LL << 30)) return MAMBA2_SCAN_EBADDIM;
  pl->NJB = SH2 / kColBlock;
  pl->V = pl->NJB * pl->NG;
  // Backward slices: about kBwdTargetGroups work-groups over the V variants,
  // each slice at least one unit per wave.  Several state groups take step
  // pairs (ceil(K/2) units and the readout per sample block).
  const bool paired = pl->NG > 1;
  const int waves = paired ? kBwdPairWaves : kBwdWaves;
  const int units = pl->NB * (paired ? (K + 1) / 2 + 1 : K + 1);
  int p0 = (kBwdTargetGroups + pl->V - 1) / pl->V;
  if (p0 > (units + waves - 1) / waves) p0 = (units + waves - 1) / waves;
  pl->UPW = (units + p0 - 1) / p0;
  pl->P = (units + pl->UPW - 1) / pl->UPW;
  pl->saved_bytes = (size_t)pl->NB * pl->NG * (size_t)saved_planes(K) * kPlane * sizeof(float);
  // Sized for p0 >= P slices: p0 never decreases as B grows, so neither does
  // the workspace (P itself can, when UPW steps up).
  pl->ws_bytes = (size_t)pl->NG * p0 * (size_t)SH2 * 3 * kGroup * sizeof(float);
  return MAMBA2_SCAN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int launch_status() {
  return hipGetLastError() == hipSuccess ? MAMBA2_SCAN_OK : MAMBA2_SCAN_EHIP;
}

// History chunks for the forward: with few sample blocks and a long history
// the chunks of one block run in parallel (a summary pass, the carry, then
// the full pass per chunk).  Chunks are whole pairs of rounds, and the last
// one spans at least two rounds (its summary needs two S planes).
void fwd_chunks(const Plan& pl, int* L, int* C) {
  *L = pl.K;
  *C = 1;
  const long long wgs = (long long)pl.NB * pl.NG;
  if (pl.K < 4 * kChunk || wgs >= kFwdChunkTarget / 2) return;
  long long c = (kFwdChunkTarget + wgs - 1) / wgs;
  if (c > pl.K / (2 * kChunk)) c = pl.K / (2 * kChunk);
  if (c < 2) return;
  int l = (int)((pl.K + c - 1) / c);
  l = ((l + 2 * kChunk - 1) / (2 * kChunk)) * (2 * kChunk);
  int cc = (pl.K + l - 1) / l;
  if (pl.K - (cc - 1) * l <= kChunk) cc -= 1;
  if (cc < 2) return;
  *L = l;
  *C = cc;
}

// The forward's launches for a shape, in order: what launch_fwd enqueues and
// mamba2_scan_fwd_plan reports.  Returns the count (1 or 3).
//  * C == 1: one full pass (projections, scan, saved terms, context).
//  * C > 1 (chunked history): a summary pass, the carry across chunks, then
//    the replay pass.
// Work-groups hold one or two sample blocks: two from SH2 = 320 on
// (fwd_blocks), except where two-block work-groups would leave CUs idle,
// when a full or summary pass takes one block each (4096 samples at
// SH2 = 320/512: forward 18 -> 14 / 23 -> 19 us; with every CU busy the
// two-block form is faster: 8192 samples 34 vs 38 us).  The replay pass
// always takes fwd_blocks(SH2/16) blocks.
int fwd_plan(const Plan& pl, mamba2_scan_launch* out) {
  int L, C;
  fwd_chunks(pl, &L, &C);
  const int nkc = pl.SH2 / 16;
  const int nblk = fwd_blocks(nkc);
  const int pairs = (pl.NB + nblk - 1) / nblk;
  const bool lone = nblk == 2 && (long long)pairs * pl.NG * C < kCUs;
  const int first_blk = lone ? 1 : nblk;
  const int first_units = lone ? pl.NB : pairs;
  auto set = [&](mamba2_scan_launch& l, int kernel, int blocks, int pass, int grid, int threads) {
    l.kernel = kernel;
    l.sample_blocks = blocks;
    l.pass = pass;
    l.chunks = C;
    l.chunk_steps = L;
    l.grid = grid;
    l.threads = threads;
  };
  set(out[0], MAMBA2_SCAN_KERNEL_FWD, first_blk, C == 1 ? MAMBA2_SCAN_PASS_FULL : MAMBA2_SCAN_PASS_SUMMARY,
      8 * pl.NG * ((first_units * C + 7) / 8), first_blk * kFwdWaves * 64);
  if (C == 1) return 1;
  const int nseg = carry_segments(C);  // C <= kFwdChunkTarget, so nseg <= kFwdChunkTarget / kCarrySeg
  set(out[1], MAMBA2_SCAN_KERNEL_CARRY, 0, MAMBA2_SCAN_PASS_CARRY, pl.NB * pl.NG * nseg, kCarryThreads);
  set(out[2], MAMBA2_SCAN_KERNEL_FWD, nblk, MAMBA2_SCAN_PASS_REPLAY, 8 * pl.NG * ((pairs * C + 7) / 8),
      nblk * kFwdWaves * 64);
  return 3;
}

template <int NKC, class T>
void launch_fwd(const Plan& pl, const T* H, const T* hs2, const float* WA, const float* WB,
                const float* WC, const float* stab, float* ctx, float* saved, hipStream_t st,
                const float* tw, float* he) {
  mamba2_scan_launch ls[3];
  const int n = fwd_plan(pl, ls);
  for (int i = 0; i < n; ++i) {
    const mamba2_scan_launch& l = ls[i];
    const dim3 grid(l.grid), block(l.threads);
    // the blend rides on the pass that writes context
    const bool last = l.pass == MAMBA2_SCAN_PASS_FULL || l.pass == MAMBA2_SCAN_PASS_REPLAY;
    const float* twp = last ? tw : nullptr;
    float* hep = last ? he : nullptr;
    if (l.kernel == MAMBA2_SCAN_KERNEL_CARRY) {
      hipLaunchKernelGGL(fwd_carry_kernel, grid, block, 0, st, pl.NB * pl.NG, pl.K, l.chunk_steps, l.chunks,
                         l.grid / (pl.NB * pl.NG), saved);
    } else if (l.pass == MAMBA2_SCAN_PASS_REPLAY) {
      hipLaunchKernelGGL((fwd_kernel<NKC, T, true>), grid, block, 0, st, pl.B, pl.K, pl.NG, pl.NB, H, hs2, WA, WB,
                         WC, stab, ctx, saved, l.chunk_steps, l.chunks, 2, twp, hep);
    } else if (l.sample_blocks == 1) {
      hipLaunchKernelGGL((fwd_kernel<NKC, T, false, 1>), grid, block, 0, st, pl.B, pl.K, pl.NG, pl.NB, H, hs2, WA,
                         WB, WC, stab, ctx, saved, l.chunk_steps, l.chunks, l.pass == MAMBA2_SCAN_PASS_FULL ? 0 : 1,
                         twp, hep);
    } else if constexpr (fwd_blocks(NKC) == 2) {
      hipLaunchKernelGGL((fwd_kernel<NKC, T, false, 2>), grid, block, 0, st, pl.B, pl.K, pl.NG, pl.NB, H, hs2, WA,
                         WB, WC, stab, ctx, saved, l.chunk_steps, l.chunks, l.pass == MAMBA2_SCAN_PASS_FULL ? 0 : 1,
                         twp, hep);
    }
  }
}

// Several state groups: the backward addresses a 16-sample block's rows with
// 32-bit buffer offsets, so they must span less than 4 GiB.
bool bwd_rows_fit(const Plan& pl) { return pl.NG == 1 || (long long)pl.K * pl.SH2 <= kDinMaxRowFloats; }

int check_bwd_common(const Plan& pl, const void* H, const void* hs2, const void* saved, size_t saved_bytes,
                     const float* dctx, const float* da, const float* db, const float* dc, const void* ws,
                     size_t ws_bytes) {
  if (!bwd_rows_fit(pl)) return MAMBA2_SCAN_EUNSUPPORTED;
  if (!H || !hs2 || !saved || !dctx || !ws) return MAMBA2_SCAN_ENULL;
  if (saved_bytes < pl.saved_bytes || ws_bytes < pl.ws_bytes) return MAMBA2_SCAN_ESIZE;
  if (!aligned16(H) || !aligned16(hs2) || !aligned16(saved) || !aligned16(ws) || !aligned4(dctx))
    return MAMBA2_SCAN_EALIGN;
  if ((da && !aligned4(da)) || (db && !aligned4(db)) || (dc && !aligned4(dc))) return MAMBA2_SCAN_EALIGN;
  return MAMBA2_SCAN_OK;
}

int check_reduce(const Plan& pl, const void* ws, size_t ws_bytes, const float* dWA, const float* dWB,
                 const float* dWC) {
  if (!ws || !dWA || !dWB || !dWC) return MAMBA2_SCAN_ENULL;
  if (ws_bytes < pl.ws_bytes) return MAMBA2_SCAN_ESIZE;
  if (!aligned16(ws) || !aligned4(dWA) || !aligned4(dWB) || !aligned4(dWC)) return MAMBA2_SCAN_EALIGN;
  return MAMBA2_SCAN_OK;
}

// din: the input gradients in the same launch (STATE_D = 16 only; no debug
// outputs), from W_A/W_B/W_C into dH / dhs2.
template <class T>
void launch_partials(const Plan& pl, const T* H, const T* hs2, const void* saved, const float* dctx,
                     float* da, float* db, float* dc, void* ws, hipStream_t st, bool din = false,
                     const float* WA = nullptr, const float* WB = nullptr, const float* WC = nullptr,
                     float* dH = nullptr, float* dhs2 = nullptr) {
  const int grid = 8 * pl.V * ((pl.P + 7) / 8);
  const bool dbg = da || db || dc, rounds = pl.K > kChunk;
  constexpr int NWD = sizeof(T) == 4 ? 8 : kBwdWaves;  // waves of the DIN form
  // several state groups: step pairs on bf16 matrix cores, history tiles
  // shared through L2
  const bool paired = pl.NG > 1;
  constexpr int NWP = kBwdPairWaves;
  auto kern = din ? (rounds ? bwd_partials_kernel<T, false, true, true, NWD>
                            : bwd_partials_kernel<T, false, false, true, NWD>)
              : paired ? (dbg ? (rounds ? bwd_partials_kernel<T, true, true, false, NWP, true>
                                        : bwd_partials_kernel<T, true, false, false, NWP, true>)
                              : (rounds ? bwd_partials_kernel<T, false, true, false, NWP, true>
                                        : bwd_partials_kernel<T, false, false, false, NWP, true>))
              : dbg ? (rounds ? bwd_partials_kernel<T, true, true> : bwd_partials_kernel<T, true, false>)
                    : (rounds ? bwd_partials_kernel<T, false, true> : bwd_partials_kernel<T, false, false>);
  const int threads = (din ? NWD : paired ? NWP : kBwdWaves) * 64;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, st, pl.B, pl.K, pl.SH2, pl.NG,
                     pl.NB, pl.P, pl.UPW, H, hs2, static_cast<const float*>(saved), dctx, da, db, dc,
                     static_cast<float*>(ws), WA, WB, WC, dH, dhs2);
}

void launch_reduce(const Plan& pl, const void* ws, float* dWA, float* dWB, float* dWC, hipStream_t st,
                   int Pw = 0, const float* wsw = nullptr, float* dw = nullptr) {
  const int quads = pl.NG * pl.SH2 * 3 * kGroup / 4;
  int grid = (quads + kRedQuads - 1) / kRedQuads;
  if (dw != nullptr) grid += (pl.SH2 / 4 + kRedQuads - 1) / kRedQuads;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(grid), dim3(kRedThreads), 0, st, pl.SH2, pl.NG, pl.P,
                     static_cast<const float*>(ws), dWA, dWB, dWC, Pw, wsw, dw);
}

int check_fwd(const Plan& pl, const void* H, const void* hs2, const float* WA, const float* WB, const float* WC,
              const float* ctx, const void* saved, size_t saved_bytes) {
  if (!H || !hs2 || !WA || !WB || !WC || !ctx || !saved) return MAMBA2_SCAN_ENULL;
  if (saved_bytes < pl.saved_bytes) return MAMBA2_SCAN_ESIZE;
  if (!aligned16(H) || !aligned16(hs2) || !aligned16(saved) || !aligned16(WA) || !aligned16(WB) ||
      !aligned16(WC) || !aligned4(ctx))
    return MAMBA2_SCAN_EALIGN;
  return MAMBA2_SCAN_OK;
}

template <class T>
int run_fwd(const Plan& pl, const T* H, const T* hs2, const float* WA, const float* WB, const float* WC,
            const float* stab, float* ctx, void* saved, hipStream_t s, const float* tw = nullptr,
            float* he = nullptr) {
  float* sv = static_cast<float*>(saved);
  switch (pl.SH2 / 64) {
    case 1: launch_fwd<4, T>(pl, H, hs2, WA, WB, WC, stab, ctx, sv, s, tw, he); break;
    case 2: launch_fwd<8, T>(pl, H, hs2, WA, WB, WC, stab, ctx, sv, s, tw, he); break;
    case 3: launch_fwd<12, T>(pl, H, hs2, WA, WB, WC, stab, ctx, sv, s, tw, he); break;
    case 4: launch_fwd<16, T>(pl, H, hs2, WA, WB, WC, stab, ctx, sv, s, tw, he); break;
    case 5: launch_fwd<20, T>(pl, H, hs2, WA, WB, WC, stab, ctx, sv, s, tw, he); break;
    case 6: launch_fwd<24, T>(pl, H, hs2, WA, WB, WC, stab, ctx, sv, s, tw, he); break;
    case 7: launch_fwd<28, T>(pl, H, hs2, WA, WB, WC, stab, ctx, sv, s, tw, he); break;
    case 8: launch_fwd<32, T>(pl, H, hs2, WA, WB, WC, stab, ctx, sv, s, tw, he); break;
    default: return MAMBA2_SCAN_EUNSUPPORTED;
  }
  return launch_status();
}

void launch_blend_fwd(const Plan& pl, const float* ctx, const float* hs2, const float* w, float* he, hipStream_t st) {
  const int grid = (pl.B + kBlendWaves - 1) / kBlendWaves;
  hipLaunchKernelGGL(blend_fwd_kernel, dim3(grid), dim3(kBlendWaves * 64), 0, st, pl.B, pl.SH2, pl.D, ctx, hs2, w,
                     he);
}

// Samples per blend-backward work-group: a multiple of its 8 waves, so that
// at most kBlendSlices work-groups (and d_temporal_weight slices) cover B.
int blend_rows_per_wg(int B) {
  const int per = (B + kBlendSlices - 1) / kBlendSlices;
  const int r = ((per + kBlendWaves - 1) / kBlendWaves) * kBlendWaves;
  return r < kBlendWaves ? kBlendWaves : r;
}

size_t blend_ws_offset(const Plan& pl) { return (pl.ws_bytes + 255) & ~(size_t)255; }
size_t blend_ws_bytes(const Plan& pl) {
  return blend_ws_offset(pl) + (size_t)kBlendSlices * pl.SH2 * sizeof(float);
}

// Units per work-group: the (block, t) units of all blocks, in order, split
// into slices so that about kDinTargetWGs work-groups run (twice as many when
// K spans several rounds: K = 64 and long_few ran 3 % faster, the pages'
// shape 5 % slower), at least one unit per wave, whatever the mix of samples
// and history length.  One state group: at most one batch of units per wave
// (more work-groups, up to kDinMaxWGs).
int dinput_upw(const Plan& pl) {
  const long long units = (long long)pl.NB * (pl.K + 1);
  const int target = pl.K > kChunk ? kDinTargetWGsRounds : kDinTargetWGs;
  const long long slices = (target + pl.NJB - 1) / pl.NJB;
  long long upw = (units + slices - 1) / slices;
  if (upw < kDinWaves) upw = kDinWaves;
  if (pl.NG == 1) {
    // one batch per wave where at most kDinMaxWGs work-groups do it
    const long long fit = (units * pl.NJB + kDinMaxWGs - 1) / kDinMaxWGs;
    const long long cap = fit > kDinBatch * kDinWaves ? fit : kDinBatch * kDinWaves;
    if (upw > cap) upw = cap;
  }
  return (int)(upw > units ? units : upw);
}

template <int NGT>
void launch_dinput(const Plan& pl, const float* WA, const float* WB, const float* WC, const float* sv,
                   const float* dctx, float* dH, float* dhs2, hipStream_t st) {
  const int upw = dinput_upw(pl);
  const long long units = (long long)pl.NB * (pl.K + 1);
  const int nsl = (int)((units + upw - 1) / upw);
  const int grid = 8 * pl.NJB * ((nsl + 7) / 8);
  if (pl.K > kChunk)
    hipLaunchKernelGGL((dinput_kernel<NGT, true>), dim3(grid), dim3(kDinWaves * 64), 0, st, pl.B, pl.K, pl.SH2,
                       pl.NB, upw, WA, WB, WC, sv, dctx, dH, dhs2);
  else
    hipLaunchKernelGGL((dinput_kernel<NGT, false>), dim3(grid), dim3(kDinWaves * 64), 0, st, pl.B, pl.K, pl.SH2,
                       pl.NB, upw, WA, WB, WC, sv, dctx, dH, dhs2);
}

// Scratch for callers that cannot allocate (mamba2_scan_bwd_noalloc): the
// backward's split-K slices live here instead of in a caller workspace.
// Every supported shape needs at most ~3.3 MiB of slices (about 256 slices
// of SH2 x 48 floats per state group, fewer as SH2 * STATE_D grows).  Each
// device holds its own copy until the process ends; calls on one device
// share it.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device with that device current (the host-side name is a stand-in, not a
// device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MAMBA2_SCAN_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MAMBA2_SCAN_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MAMBA2_SCAN_OK;
}

// The argument checks of mamba2_scan_bwd, less the workspace (the no-alloc
// backward brings its own): all of them run before the scratch address is
// looked up, so a bad call returns without touching the device.
int check_bwd_noalloc(const Plan& pl, const void* H, const void* hs2, const void* saved, size_t saved_bytes,
                      const float* dctx, const float* dWA, const float* dWB, const float* dWC, const float* da,
                      const float* db, const float* dc) {
  if (!bwd_rows_fit(pl)) return MAMBA2_SCAN_EUNSUPPORTED;
  if (!H || !hs2 || !saved || !dctx || !dWA || !dWB || !dWC) return MAMBA2_SCAN_ENULL;
  if (saved_bytes < pl.saved_bytes) return MAMBA2_SCAN_ESIZE;
  if (pl.ws_bytes > kScratchBytes) return MAMBA2_SCAN_ESCRATCH;
  if (!aligned16(H) || !aligned16(hs2) || !aligned16(saved) || !aligned4(dctx) || !aligned4(dWA) ||
      !aligned4(dWB) || !aligned4(dWC))
    return MAMBA2_SCAN_EALIGN;
  if ((da && !aligned4(da)) || (db && !aligned4(db)) || (dc && !aligned4(dc))) return MAMBA2_SCAN_EALIGN;
  return MAMBA2_SCAN_OK;
}

}  // namespace

extern "C" {

size_t mamba2_scan_saved_bytes(int B, int K, int SH2, int STATE_D) {
  Plan pl;
  return make_plan(B, K, SH2, STATE_D, &pl) == MAMBA2_SCAN_OK ? pl.saved_bytes : 0;
}

size_t mamba2_scan_bwd_workspace_bytes(int B, int K, int SH2, int STATE_D) {
  Plan pl;
  return make_plan(B, K, SH2, STATE_D, &pl) == MAMBA2_SCAN_OK && bwd_rows_fit(pl) ? pl.ws_bytes : 0;
}

int mamba2_scan_fwd(int B, int K, int SH2, int STATE_D, const float* h_history, const float* h_s2,
                    const float* W_A, const float* W_B, const float* W_C, float* context, void* saved,
                    size_t saved_bytes, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_fwd(pl, h_history, h_s2, W_A, W_B, W_C, context, saved, saved_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  return run_fwd(pl, h_history, h_s2, W_A, W_B, W_C, nullptr, context, saved, static_cast<hipStream_t>(stream));
}

int mamba2_scan_fwd_blend(int B, int K, int SH2, int STATE_D, const float* h_history, const float* h_s2,
                          const float* W_A, const float* W_B, const float* W_C, const float* stability,
                          const float* temporal_weight, float* context, float* h_enriched, void* saved,
                          size_t saved_bytes, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_fwd(pl, h_history, h_s2, W_A, W_B, W_C, context, saved, saved_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  if (!aligned4(stability) || !aligned16(temporal_weight) || !aligned16(h_enriched)) return MAMBA2_SCAN_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one state group: the forward kernel writes h_enriched itself
  const bool fused = pl.NG == 1 && h_enriched != nullptr;
  st = run_fwd(pl, h_history, h_s2, W_A, W_B, W_C, stability, context, saved, s, fused ? temporal_weight : nullptr,
               fused ? h_enriched : nullptr);
  if (st != MAMBA2_SCAN_OK || h_enriched == nullptr || fused) return st;
  launch_blend_fwd(pl, context, h_s2, temporal_weight, h_enriched, s);
  return launch_status();
}

int mamba2_scan_bwd_partials(int B, int K, int SH2, int STATE_D, const float* h_history, const float* h_s2,
                             const void* saved, size_t saved_bytes, const float* d_context, float* d_a, float* d_b,
                             float* d_c, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_bwd_common(pl, h_history, h_s2, saved, saved_bytes, d_context, d_a, d_b, d_c, workspace,
                        workspace_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  launch_partials(pl, h_history, h_s2, saved, d_context, d_a, d_b, d_c, workspace,
                  static_cast<hipStream_t>(stream));
  return launch_status();
}

int mamba2_scan_bwd_reduce(int B, int K, int SH2, int STATE_D, const void* workspace, size_t workspace_bytes,
                           float* dW_A, float* dW_B, float* dW_C, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_reduce(pl, workspace, workspace_bytes, dW_A, dW_B, dW_C);
  if (st != MAMBA2_SCAN_OK) return st;
  launch_reduce(pl, workspace, dW_A, dW_B, dW_C, static_cast<hipStream_t>(stream));
  return launch_status();
}

int mamba2_scan_bwd(int B, int K, int SH2, int STATE_D, const float* h_history, const float* h_s2,
                    const void* saved, size_t saved_bytes, const float* d_context, float* dW_A, float* dW_B,
                    float* dW_C, float* d_a, float* d_b, float* d_c, void* workspace, size_t workspace_bytes,
                    void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_bwd_common(pl, h_history, h_s2, saved, saved_bytes, d_context, d_a, d_b, d_c, workspace,
                        workspace_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_reduce(pl, workspace, workspace_bytes, dW_A, dW_B, dW_C);
  if (st != MAMBA2_SCAN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_partials(pl, h_history, h_s2, saved, d_context, d_a, d_b, d_c, workspace, s);
  st = launch_status();
  if (st != MAMBA2_SCAN_OK) return st;
  launch_reduce(pl, workspace, dW_A, dW_B, dW_C, s);
  return launch_status();
}

int mamba2_scan_bwd_noalloc(int B, int K, int SH2, int STATE_D, const float* h_history, const float* h_s2,
                            const void* saved, size_t saved_bytes, const float* d_context, float* dW_A, float* dW_B,
                            float* dW_C, float* d_a, float* d_b, float* d_c, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_bwd_noalloc(pl, h_history, h_s2, saved, saved_bytes, d_context, dW_A, dW_B, dW_C, d_a, d_b, d_c);
  if (st != MAMBA2_SCAN_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MAMBA2_SCAN_OK) return st;
  return mamba2_scan_bwd(B, K, SH2, STATE_D, h_history, h_s2, saved, saved_bytes, d_context, dW_A, dW_B, dW_C, d_a,
                         d_b, d_c, ws, kScratchBytes, stream);
}

int mamba2_scan_fwd_bf16(int B, int K, int SH2, int STATE_D, const void* h_history, const void* h_s2,
                         const float* W_A, const float* W_B, const float* W_C, float* context, void* saved,
                         size_t saved_bytes, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_fwd(pl, h_history, h_s2, W_A, W_B, W_C, context, saved, saved_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  return run_fwd(pl, static_cast<const bf16_t*>(h_history), static_cast<const bf16_t*>(h_s2), W_A, W_B, W_C,
                 nullptr, context, saved, static_cast<hipStream_t>(stream));
}

int mamba2_scan_bwd_partials_bf16(int B, int K, int SH2, int STATE_D, const void* h_history, const void* h_s2,
                                  const void* saved, size_t saved_bytes, const float* d_context, float* d_a,
                                  float* d_b, float* d_c, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_bwd_common(pl, h_history, h_s2, saved, saved_bytes, d_context, d_a, d_b, d_c, workspace,
                        workspace_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  launch_partials(pl, static_cast<const bf16_t*>(h_history), static_cast<const bf16_t*>(h_s2), saved, d_context,
                  d_a, d_b, d_c, workspace, static_cast<hipStream_t>(stream));
  return launch_status();
}

int mamba2_scan_bwd_bf16(int B, int K, int SH2, int STATE_D, const void* h_history, const void* h_s2,
                         const void* saved, size_t saved_bytes, const float* d_context, float* dW_A, float* dW_B,
                         float* dW_C, float* d_a, float* d_b, float* d_c, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_bwd_common(pl, h_history, h_s2, saved, saved_bytes, d_context, d_a, d_b, d_c, workspace,
                        workspace_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_reduce(pl, workspace, workspace_bytes, dW_A, dW_B, dW_C);
  if (st != MAMBA2_SCAN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_partials(pl, static_cast<const bf16_t*>(h_history), static_cast<const bf16_t*>(h_s2), saved, d_context,
                  d_a, d_b, d_c, workspace, s);
  st = launch_status();
  if (st != MAMBA2_SCAN_OK) return st;
  launch_reduce(pl, workspace, dW_A, dW_B, dW_C, s);
  return launch_status();
}

size_t mamba2_scan_bwd_blend_workspace_bytes(int B, int K, int SH2, int STATE_D) {
  Plan pl;
  return make_plan(B, K, SH2, STATE_D, &pl) == MAMBA2_SCAN_OK ? blend_ws_bytes(pl) : 0;
}

int mamba2_scan_bwd_blend(int B, int K, int SH2, int STATE_D, const float* h_history, const float* h_s2,
                          const void* saved, size_t saved_bytes, const float* temporal_weight,
                          const float* d_h_enriched, float* d_context, float* dW_A, float* dW_B, float* dW_C,
                          float* d_temporal_weight, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  if (!d_h_enriched || !d_context) return MAMBA2_SCAN_ENULL;
  st = check_bwd_common(pl, h_history, h_s2, saved, saved_bytes, d_context, nullptr, nullptr, nullptr, workspace,
                        workspace_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_reduce(pl, workspace, workspace_bytes, dW_A, dW_B, dW_C);
  if (st != MAMBA2_SCAN_OK) return st;
  if (workspace_bytes < blend_ws_bytes(pl)) return MAMBA2_SCAN_ESIZE;
  if (!aligned16(d_h_enriched) || !aligned16(temporal_weight) || !aligned4(d_temporal_weight))
    return MAMBA2_SCAN_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rpw = blend_rows_per_wg(B);
  const int pw = (B + rpw - 1) / rpw;
  float* wsw = reinterpret_cast<float*>(static_cast<char*>(workspace) + blend_ws_offset(pl));
  hipLaunchKernelGGL(blend_bwd_kernel, dim3(pw), dim3(kBlendWaves * 64), 0, s, B, K, SH2, pl.NG, rpw,
                     static_cast<const float*>(saved), temporal_weight, d_h_enriched, d_context, wsw);
  st = launch_status();
  if (st != MAMBA2_SCAN_OK) return st;
  launch_partials(pl, h_history, h_s2, saved, d_context, nullptr, nullptr, nullptr, workspace, s);
  st = launch_status();
  if (st != MAMBA2_SCAN_OK) return st;
  launch_reduce(pl, workspace, dW_A, dW_B, dW_C, s, pw, wsw, d_temporal_weight);
  return launch_status();
}

int mamba2_scan_bwd_input(int B, int K, int SH2, int STATE_D, const float* W_A, const float* W_B,
                          const float* W_C, const void* saved, size_t saved_bytes, const float* d_context,
                          float* d_h_history, float* d_h_s2, void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  // a 16-sample block's rows must span less than 4 GiB (32-bit store offsets)
  if ((long long)K * SH2 > kDinMaxRowFloats) return MAMBA2_SCAN_EUNSUPPORTED;
  if (!W_A || !W_B || !W_C || !saved || !d_context || (!d_h_history && !d_h_s2)) return MAMBA2_SCAN_ENULL;
  if (saved_bytes < pl.saved_bytes) return MAMBA2_SCAN_ESIZE;
  if (!aligned16(saved) || !aligned4(W_A) || !aligned4(W_B) || !aligned4(W_C) || !aligned4(d_context) ||
      !aligned16(d_h_history) || !aligned16(d_h_s2))
    return MAMBA2_SCAN_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* sv = static_cast<const float*>(saved);
  switch (pl.NG) {
    case 1: launch_dinput<1>(pl, W_A, W_B, W_C, sv, d_context, d_h_history, d_h_s2, s); break;
    case 2: launch_dinput<2>(pl, W_A, W_B, W_C, sv, d_context, d_h_history, d_h_s2, s); break;
    case 4: launch_dinput<4>(pl, W_A, W_B, W_C, sv, d_context, d_h_history, d_h_s2, s); break;
    default: return MAMBA2_SCAN_EUNSUPPORTED;
  }
  return launch_status();
}

int mamba2_scan_fwd_plan(int B, int K, int SH2, int STATE_D, mamba2_scan_launch* launches, int max_launches) {
  Plan pl;
  const int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  if (max_launches > 0 && launches == nullptr) return MAMBA2_SCAN_ENULL;
  mamba2_scan_launch ls[3];
  const int n = fwd_plan(pl, ls);
  for (int i = 0; i < n && i < max_launches; ++i) launches[i] = ls[i];
  return n;
}

}  // extern "C"

namespace {
// The backward with the input gradients: one pass over the history when
// STATE_D = 16, else the weight-gradient backward then the input-gradient
// kernel (the same results as the two separate calls).
template <class T>
int run_bwd_full(int B, int K, int SH2, int STATE_D, const T* H, const T* hs2, const void* saved,
                 size_t saved_bytes, const float* dctx, const float* WA, const float* WB, const float* WC,
                 float* dWA, float* dWB, float* dWC, float* dH, float* dhs2, void* ws, size_t ws_bytes,
                 void* stream) {
  Plan pl;
  int st = make_plan(B, K, SH2, STATE_D, &pl);
  if (st != MAMBA2_SCAN_OK) return st;
  // a 16-sample block's rows must span less than 4 GiB (32-bit store offsets)
  if ((long long)K * SH2 > kDinMaxRowFloats) return MAMBA2_SCAN_EUNSUPPORTED;
  st = check_bwd_common(pl, H, hs2, saved, saved_bytes, dctx, nullptr, nullptr, nullptr, ws, ws_bytes);
  if (st != MAMBA2_SCAN_OK) return st;
  st = check_reduce(pl, ws, ws_bytes, dWA, dWB, dWC);
  if (st != MAMBA2_SCAN_OK) return st;
  if (!WA || !WB || !WC || (!dH && !dhs2)) return MAMBA2_SCAN_ENULL;
  if (!aligned16(WA) || !aligned16(WB) || !aligned16(WC) || !aligned16(dH) || !aligned16(dhs2))
    return MAMBA2_SCAN_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = pl.NG == 1;
  launch_partials(pl, H, hs2, saved, dctx, nullptr, nullptr, nullptr, ws, s, fused, WA, WB, WC, dH, dhs2);
  st = launch_status();
  if (st != MAMBA2_SCAN_OK) return st;
  launch_reduce(pl, ws, dWA, dWB, dWC, s);
  st = launch_status();
  if (st != MAMBA2_SCAN_OK || fused) return st;
  const float* sv = static_cast<const float*>(saved);
  switch (pl.NG) {
    case 2: launch_dinput<2>(pl, WA, WB, WC, sv, dctx, dH, dhs2, s); break;
    case 4: launch_dinput<4>(pl, WA, WB, WC, sv, dctx, dH, dhs2, s); break;
    default: return MAMBA2_SCAN_EUNSUPPORTED;
  }
  return launch_status();
}
}  // namespace

extern "C" {

int mamba2_scan_bwd_full(int B, int K, int SH2, int STATE_D, const float* h_history, const float* h_s2,
                         const void* saved, size_t saved_bytes, const float* d_context, const float* W_A,
                         const float* W_B, const float* W_C, float* dW_A, float* dW_B, float* dW_C,
                         float* d_h_history, float* d_h_s2, void* workspace, size_t workspace_bytes, void* stream) {
  return run_bwd_full(B, K, SH2, STATE_D, h_history, h_s2, saved, saved_bytes, d_context, W_A, W_B, W_C, dW_A,
                      dW_B, dW_C, d_h_history, d_h_s2, workspace, workspace_bytes, stream);
}

int mamba2_scan_bwd_full_bf16(int B, int K, int SH2, int STATE_D, const void* h_history, const void* h_s2,
                              const void* saved, size_t saved_bytes, const float* d_context, const float* W_A,
                              const float* W_B, const float* W_C, float* dW_A, float* dW_B, float* dW_C,
                              float* d_h_history, float* d_h_s2, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return run_bwd_full(B, K, SH2, STATE_D, static_cast<const bf16_t*>(h_history), static_cast<const bf16_t*>(h_s2),
                      saved, saved_bytes, d_context, W_A, W_B, W_C, dW_A, dW_B, dW_C, d_h_history, d_h_s2, workspace,
                      workspace_bytes, stream);
}

const char* mamba2_scan_strerror(int status) {
  switch (status) {
    case MAMBA2_SCAN_OK: return "success";
    case MAMBA2_SCAN_EBADDIM: return "invalid dimension (must be > 0 and sizes must not overflow)";
    case MAMBA2_SCAN_EUNSUPPORTED: return "unsupported shape (STATE_D in {16,32,64}; SH2 % 64 == 0, SH2 <= 512)";
    case MAMBA2_SCAN_ENULL: return "a required pointer is NULL";
    case MAMBA2_SCAN_ESIZE: return "saved or workspace buffer is smaller than required";
    case MAMBA2_SCAN_EALIGN: return "pointer misaligned (inputs, saved and workspace need 16 bytes)";
    case MAMBA2_SCAN_EHIP: return "HIP runtime error while enqueuing a kernel";
    case MAMBA2_SCAN_ESCRATCH: return "the shape needs more scratch than the library's fixed 4 MiB buffer";
    default: return "unknown status";
  }
}

}  // extern "C"
