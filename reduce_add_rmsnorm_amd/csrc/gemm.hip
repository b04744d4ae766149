// gemm.hip -- the producer of the shard path: one rank's row-parallel GEMM
// with its ReduceScatter destinations (include/sprms.h, sp_matmul_scatter).
//
// Rank q computes P = x w^T, x [M][K] and w [N][K] in bf16 (both operands
// K-contiguous, the layout of a linear layer's weight), fp32 accumulation on
// the matrix cores, and writes token row m straight into slot q of rank
// m / S's [tp][S][N] receive buffer -- the buffer the fused reduce + add +
// RMSNorm kernel consumes.  On one GPU the receive buffers are local; on a
// node they would be peer-mapped and this epilogue is the "send each block as
// soon as it is computed" half of a fused GEMM + ReduceScatter.
//
// Kernel design (gfx950, dense bf16: MFMA bound at the shapes of interest,
// e.g. 2*65536*896*7168 flop against 1.07 GB at C4's shape, 785 flop/B, above
// the 312 flop/B ridge of 2.5 PFLOP/s over 8 TB/s):
//   * one workgroup of 8 wavefronts per 256 x 256 output tile, two
//     wavefronts per SIMD so that one issues MFMAs while the other waits on
//     LDS or a barrier; each wavefront owns 128 columns x 64 tokens (128 fp32
//     accumulators per lane): bf16 as 8 x 4 blocks of
//     v_mfma_f32_16x16x32_bf16 (measured ~4% faster than 4 x 2 blocks of the
//     32x32x16 form with the same LDS traffic), e4m3 as 4 x 2 blocks of
//     v_mfma_scale_f32_32x32x64_f8f6f4;
//   * the weight tile is the MFMA's A operand and the token tile its B
//     operand, so each lane's accumulators are 4-element runs of one token
//     row's output columns;
//   * K advances 128 bytes of each row at a time (64 bf16 or 128 e4m3
//     elements) through two LDS stages filled by buffer loads that write LDS
//     directly (16 bytes per lane, no staging registers).  bf16 is
//     software-pipelined: a stage's fragments are all in registers when its
//     step begins, each is refilled from the next stage right after its last
//     MFMA, and the loads two stages ahead are spread over the first k-step
//     (6-8% faster than reading each k-step's fragments at its start, which
//     left every wavefront waiting on LDS at each barrier).  e4m3 issues the
//     next stage's loads before the current stage's MFMAs and reads
//     fragments per k-step (the pipelined form was slower there).  LDS rows
//     are 128 bytes with their 16-byte chunks XOR-swizzled by (row >> 1) & 7,
//     so the 16 rows an MFMA operand read touches per 16 lanes land on
//     distinct banks;
//   * the epilogue stages the rounded tile in LDS and writes each token row
//     as 512 contiguous bytes (16 per lane): written from the accumulator
//     layout directly, every 8-byte piece became its own DRAM write, 4x the
//     output bytes;
//   * tiles are ordered for the L2 of each XCD: workgroup b runs on XCD b % 8,
//     each XCD gets a contiguous range of tile ids, and tile ids run over
//     groups of 4 token bands x all column tiles, so the ~32 tiles resident
//     on an XCD share their token bands and weight tiles;
//   * tails: loads through per-tile buffer descriptors return 0 past the last
//     row; chunks at or past K (K % 8 == 0) are given an offset past the
//     descriptor, which also reads 0; stores are skipped past M and N.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "common.h"
#include "sprms.h"

namespace {

using namespace sprms;

constexpr int kBM = 256;                 // token rows per tile
constexpr int kBN = 256;                 // output columns per tile
constexpr int kBK = 64;                  // K per LDS stage
constexpr int kThreads = 512;            // 8 wavefronts
constexpr int kOpBytes = kBM * kBK * 2;  // one operand of one stage: 256 rows x 128 bytes
constexpr int kStageBytes = 2 * kOpBytes;
// epilogue staging: a bf16 tile (256 rows of 512 bytes + 16 of padding) at
// once, an f32 tile in two passes of 128 rows of 1 KiB + 16
constexpr int kOutRowsF32 = 128;
constexpr int out_row_bytes(int esz) { return kBN * esz + 16; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kSmemBytes = cmax(2 * kStageBytes, cmax(kBM * out_row_bytes(2), kOutRowsF32 * out_row_bytes(4)));
constexpr int kGroupM = 4;               // token bands per tile group
constexpr int kXcds = 8;
// s_waitcnt operand that waits for lgkmcnt(0) only (vmcnt and expcnt at their maxima)
constexpr int kLgkmZero = 0xC07F;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct MArgs {
  const char* x;            // [M][K] bf16 or e4m3
  const char* w;            // [N][K] bf16 or e4m3
  const float* x_scale;     // e4m3 inputs: 1 or M entries (per tensor / per token)
  const float* w_scale;     // e4m3 inputs: 1 or N entries (per tensor / per column)
  char* dst[kMaxTp];        // rank r's [tp][S][N] receive buffer
  int64_t S;
  int64_t slot;             // rank * S: first row of this rank's slot
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t x_scale_rows, w_scale_rows;
};

// tile id of workgroup b: XCD-contiguous ranges over a grouped order
__device__ __forceinline__ void tile_of(const MArgs& a, int* tm, int* tn) {
  const int total = a.tiles_m * a.tiles_n;
  const int b = blockIdx.x;
  const int x = b % kXcds, i = b / kXcds;
  const int q = total / kXcds, rem = total % kXcds;
  const int t = x * q + (x < rem ? x : rem) + i;
  const int per_group = kGroupM * a.tiles_n;
  const int g = t / per_group;
  const int first = g * kGroupM;
  const int gm = a.tiles_m - first < kGroupM ? a.tiles_m - first : kGroupM;
  const int in = t - g * per_group;
  *tm = first + in % gm;
  *tn = in / gm;
}

// physical 16-byte chunk of logical chunk c in LDS row `row`
__device__ __forceinline__ int swizzle(int row, int c) { return c ^ ((row >> 1) & 7); }

// IN: SP_BF16 (v_mfma_f32_16x16x32_bf16, K 32 a step) or SP_FP8_E4M3
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales, K 64 a step,
// the input scales applied in the epilogue).  Either way an LDS row is 128
// bytes per stage: 64 bf16 or 128 e4m3 elements of K.
//
// Block geometry (BLK = 16 or 32 rows and columns per MFMA block): lane l
// reads operand row l % BLK of each block, and the 64 / BLK lane groups split
// the step's K chunks among them; accumulator element 4g + c of block (i, j)
// is output column BLK*i + 8g + 4*(l / BLK) + c of token BLK*j + l % BLK
// (g < BLK * BLK / 256).
template <int OUT, int IN>
__global__ void __launch_bounds__(kThreads) matmul_scatter_kernel(const MArgs a) {
  constexpr bool fp8 = IN == SP_FP8_E4M3;
  constexpr int E = fp8 ? 1 : 2;                 // input bytes per element
  constexpr int BK = kBK * 2 / E;                // K elements per stage
  constexpr int KSTEP = fp8 ? 64 : 32;           // K elements per MFMA
  constexpr int BLK = fp8 ? 32 : 16;             // MFMA block rows / columns
  constexpr int NI = 128 / BLK, NJ = 64 / BLK;   // blocks per wavefront: columns x tokens
  constexpr int RUNS = BLK * BLK / 256;          // 4-column runs per lane and block: 1 or 4
  typedef float Acc __attribute__((ext_vector_type(BLK * BLK / 64)));
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  int tm, tn;
  tile_of(a, &tm, &tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x;
  // wave-uniform in a scalar register, so that the LDS destinations of the
  // direct-to-LDS loads (M0) are scalar arithmetic, not a VALU result read
  // back per load
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // tokens [wm*64, +64), columns [wn*128, +128)

  // per-tile descriptors: rows past M (N) read as zero
  const uint32_t row_bytes = static_cast<uint32_t>(a.K) * E;
  const int rows_x = a.M - m0 < kBM ? a.M - m0 : kBM;
  const int rows_w = a.N - n0 < kBN ? a.N - n0 : kBN;
  const rsrc_t gx = row_rsrc(a.x + static_cast<int64_t>(m0) * row_bytes, static_cast<uint32_t>(rows_x) * row_bytes);
  const rsrc_t gw = row_rsrc(a.w + static_cast<int64_t>(n0) * row_bytes, static_cast<uint32_t>(rows_w) * row_bytes);

  // One load instruction of a wavefront fills 1 KiB of LDS: 8 rows x 128
  // bytes, lane l at byte 16*l, i.e. row l >> 3, physical chunk l & 7; the
  // lane fetches the logical chunk that the swizzle puts there.
  const int grow = lane >> 3, pchunk = lane & 7;
  // load u (0..7) of the eight a wavefront issues per stage: rows group
  // wave + 8 * (u / 2) of the weight (u even) or token (u odd) operand
  auto issue_one = [&](int stage, int kb, int u) {
    const int g = wave + (kThreads / 64) * (u >> 1);  // group of 8 rows
    const int row = g * 8 + grow;
    const int k = kb + swizzle(row, pchunk) * (16 / E);  // first element of the chunk
    const uint32_t oob = (static_cast<uint32_t>(k - a.K) >> 31) ? 0u : 0x80000000u;
    const uint32_t off = (static_cast<uint32_t>(row) * row_bytes + static_cast<uint32_t>(k) * E) | oob;
    char* base = smem + stage * kStageBytes + g * 1024 + (u & 1) * kOpBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds((u & 1) ? gx : gw, (lds_void*)base, 16, off, 0, 0, kCachedPolicy);
  };
  constexpr int kLoads = 2 * kBM / 8 / (kThreads / 64);
  auto issue = [&](int stage, int kb) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) issue_one(stage, kb, u);
  };

  Acc acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < BLK * BLK / 64; ++e) acc[i][j][e] = 0.0f;

  const int nk = (a.K + BK - 1) / BK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // operand rows of this lane: row l % BLK of each block; lane group l / BLK
  // takes its share of each MFMA step's K chunks (bf16: one 16-byte chunk;
  // e4m3: two)
  const int arow = wn * 128 + lane % BLK, brow = wm * 64 + lane % BLK;
  const int kgrp = lane / BLK;
  constexpr int kStepChunks = KSTEP * E / 16;            // 16-byte chunks per MFMA step
  constexpr int kChunks = kStepChunks / (64 / BLK);      // chunks per lane and step: 1 or 2
  auto frag = [&](const char* op, int r, int ks) {
    const int c = ks * kStepChunks + kgrp * kChunks;
    if constexpr (fp8) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(op + r * 128 + swizzle(r, c) * 16);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(op + r * 128 + swizzle(r, c + 1) * 16);
      const i32x8 v = {static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                       static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                       static_cast<int>(hi[2]), static_cast<int>(hi[3])};
      return v;
    } else {
      return *reinterpret_cast<const bf16x8*>(op + r * 128 + swizzle(r, c) * 16);
    }
  };
  using Frag = decltype(frag(smem, 0, 0));
  auto mfma = [&](const Frag& x, const Frag& y, Acc& c) {
    if constexpr (fp8) {
      // format 0 (e4m3) for both operands, block scales 2^0 (E8M0 code 127)
      c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 127, 0, 127);
    } else {
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
    }
  };
  if constexpr (fp8) {
    // e4m3: each k-step's fragments are read at the start of the step, and
    // the loads of stage kt + 1 issued ahead of stage kt's MFMAs
    for (int kt = 0; kt < nk; ++kt) {
      // the next step's loads (past K on the last step: zeros into the idle stage)
      issue((kt + 1) & 1, (kt + 1) * BK);
      const char* sw = smem + (kt & 1) * kStageBytes;
      const char* sx = sw + kOpBytes;
#pragma unroll
      for (int ks = 0; ks < BK / KSTEP; ++ks) {
        Frag fa[NI], fb[NJ];
#pragma unroll
        for (int i = 0; i < NI; ++i) fa[i] = frag(sw, arow + i * BLK, ks);
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb[j] = frag(sx, brow + j * BLK, ks);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) mfma(fa[i], fb[j], acc[i][j]);
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wavefront's loads into the next stage have landed
      __syncthreads();
    }
  } else {
    // bf16: software-pipelined.  Both k-steps' fragments of stage kt are in
    // registers when its step starts; during the step every fragment is
    // refilled from stage kt + 1 as soon as its last MFMA has been issued
    // (an A row after its NJ MFMAs, the B fragments within the last row),
    // and the loads of stage kt + 2 go out one per A row of the first
    // k-step.  The only LDS wait left at a barrier is for the last one or
    // two reads, where reading all fragments at the start of a step left
    // every wavefront of the CU waiting for 12 reads at once.  Scheduling
    // groups keep that order: MFMA, global load, LDS read.
    static_assert(BK / KSTEP == 2 && kLoads == NI, "two k-steps per stage, one load per A row");
    Frag fa[NI], fb[NJ], na[NI], nb[NJ];  // k-step 0 and k-step 1 of the current stage
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      fa[i] = frag(smem, arow + i * BLK, 0);
      na[i] = frag(smem, arow + i * BLK, 1);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      fb[j] = frag(smem + kOpBytes, brow + j * BLK, 0);
      nb[j] = frag(smem + kOpBytes, brow + j * BLK, 1);
    }
    if (nk > 1) issue(1, BK);
    __builtin_amdgcn_s_waitcnt(kLgkmZero);
    // one stage; ISSUE: load stage kt + 2 into stage kt's buffer, NEXT: refill from stage kt + 1
    auto step = [&](int kt, auto issue_c, auto next_c) {
      constexpr bool ISSUE = decltype(issue_c)::value, NEXT = decltype(next_c)::value;
      // stage kt + 1 has landed and every wavefront has read stage kt
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const char* nx = smem + ((kt + 1) & 1) * kStageBytes;
      auto kstep = [&](Frag* A, Frag* B, int h, auto loads_c) {
        constexpr bool LOADS = decltype(loads_c)::value;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            mfma(A[i], B[j], acc[i][j]);
            if (i == NI - 1) {  // the last use of B[j]
              if constexpr (NEXT) B[j] = frag(nx + kOpBytes, brow + j * BLK, h);
              __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
              if constexpr (NEXT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
          }
          if constexpr (LOADS) issue_one(kt & 1, (kt + 2) * BK, i);
          if constexpr (NEXT) A[i] = frag(nx, arow + i * BLK, h);
          if (i < NI - 1) __builtin_amdgcn_sched_group_barrier(kSchedMfma, NJ, 0);
          if constexpr (LOADS) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
          if constexpr (NEXT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
      };
      kstep(fa, fb, 0, std::integral_constant<bool, ISSUE>{});
      kstep(na, nb, 1, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    };
    using Yes = std::true_type;
    using No = std::false_type;
    int kt = 0;
    for (; kt + 2 < nk; ++kt) step(kt, Yes{}, Yes{});
    if (kt + 1 < nk) step(kt++, No{}, Yes{});
    step(kt, No{}, No{});
    __syncthreads();  // every wavefront is done with the loop's LDS
  }

  // Epilogue: acc[i][j][4g + c] is output (token ml, column nl + c) with
  // ml = wm*64 + BLK*j + l%BLK, nl = wn*128 + BLK*i + 8g + 4*(l/BLK).  The rounded
  // tile goes through LDS (bf16: all 256 rows at once; f32: 128 rows per
  // pass), then each token row leaves as 16 bytes per lane.
  constexpr int esz = OUT == SP_F32 ? 4 : 2;
  constexpr int rows_per_pass = OUT == SP_F32 ? kOutRowsF32 : kBM;
  constexpr int lanes_per_row = kBN * esz / 16;  // 32 (bf16) or 64 (f32)
  constexpr int out_row = out_row_bytes(esz);
#pragma unroll
  for (int pass = 0; pass < kBM / rows_per_pass; ++pass) {
    if (pass > 0) __syncthreads();  // the previous pass's rows have been read
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ml = wm * 64 + j * BLK + lane % BLK - pass * rows_per_pass;
      if (ml < 0 || ml >= rows_per_pass) continue;
      float sx = 1.0f;
      if constexpr (fp8) {  // token scale; rows past M (not stored) read entry 0
        const int m = m0 + pass * rows_per_pass + ml;
        sx = a.x_scale[a.x_scale_rows == 1 || m >= a.M ? 0 : m];
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < RUNS; ++g) {
          const int nl = wn * 128 + i * BLK + g * 8 + (lane / BLK) * 4;
          float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
          float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if constexpr (fp8) {  // column scales; columns past N (not stored) read entry 0
            const int n = n0 + nl;
            const bool per_col = a.w_scale_rows != 1 && n < a.N;
            const float* sw = a.w_scale + (per_col ? n : 0);
            v0 = v0 * sx * sw[0];
            v1 = v1 * sx * sw[per_col ? 1 : 0];
            v2 = v2 * sx * sw[per_col ? 2 : 0];
            v3 = v3 * sx * sw[per_col ? 3 : 0];
          }
          char* dst = smem + ml * out_row + nl * esz;
          if constexpr (OUT == SP_F32) {
            const f32x4 v = {v0, v1, v2, v3};
            *reinterpret_cast<f32x4*>(dst) = v;
          } else {
            const f32x2 lo = {v0, v1}, hi = {v2, v3};
            const u32x2 v = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                             __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
            *reinterpret_cast<u32x2*>(dst) = v;
          }
        }
    }
    __syncthreads();
    const int col = (tid % lanes_per_row) * 16;  // byte offset in the row segment
    const bool col_ok = n0 + col / esz < a.N;    // N % 8 == 0: a 16-byte piece is all in or all out
    for (int rr = tid / lanes_per_row; rr < rows_per_pass; rr += kThreads / lanes_per_row) {
      const int m = m0 + pass * rows_per_pass + rr;
      if (m >= a.M || !col_ok) continue;
      const uint32_t r = static_cast<uint32_t>(m) / static_cast<uint32_t>(a.S);
      const int64_t s = m - static_cast<int64_t>(r) * a.S;
      char* row = a.dst[r] + ((a.slot + s) * static_cast<int64_t>(a.N) + n0) * esz;
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + rr * out_row + col);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(row + col));
    }
  }
}

// Validation and launch shared by both entry points; x_scale / w_scale are
// NULL for bf16 inputs.
int launch_matmul(const sp_matmul_problem* p, const void* x, const float* x_scale, const void* w,
                  const float* w_scale, void* const* dst, void* stream) {
  const bool fp8 = p->in_dtype == SP_FP8_E4M3;
  const int tp = p->tp;
  if (tp < 1 || tp > kMaxTp) return fail(SP_ERR_SHAPE, "tp=%d outside [1, %d]", tp, kMaxTp);
  if (p->rank < 0 || p->rank >= tp) return fail(SP_ERR_SHAPE, "rank=%d outside [0, %d)", p->rank, tp);
  if (p->out_dtype != SP_BF16 && p->out_dtype != SP_F32)
    return fail(SP_ERR_DTYPE, "out_dtype=%d must be SP_BF16 or SP_F32", p->out_dtype);
  const int64_t S = p->shard_rows, K = p->k, N = p->n;
  // bound S before multiplying, so that tp*S cannot wrap past the check
  if (S < 0 || S > INT32_MAX / tp) return fail(SP_ERR_SHAPE, "shard_rows=%lld: need 0 <= tp*S < 2^31", (long long)S);
  const int64_t M = S * tp;
  const int64_t kq = fp8 ? 16 : 8;  // K elements per 16-byte chunk
  if (K < kq || K % kq != 0 || K > (1 << 20))
    return fail(SP_ERR_SHAPE, "k=%lld must be a multiple of %lld in [%lld, 2^20]", (long long)K, (long long)kq,
                (long long)kq);
  if (N < 8 || N % 8 != 0 || N > (1 << 20))
    return fail(SP_ERR_SHAPE, "n=%lld must be a multiple of 8 in [8, 2^20]", (long long)N);
  if (fp8) {
    if (p->x_scale_rows != 1 && p->x_scale_rows != M)
      return fail(SP_ERR_SHAPE, "x_scale_rows=%lld must be 1 or M=%lld", (long long)p->x_scale_rows, (long long)M);
    if (p->w_scale_rows != 1 && p->w_scale_rows != N)
      return fail(SP_ERR_SHAPE, "w_scale_rows=%lld must be 1 or N=%lld", (long long)p->w_scale_rows, (long long)N);
  } else if (p->x_scale_rows != 0 || p->w_scale_rows != 0) {
    return fail(SP_ERR_SHAPE, "bf16 inputs take no scales (x_scale_rows and w_scale_rows must be 0)");
  }
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (tiles > INT32_MAX) return fail(SP_ERR_SHAPE, "too many tiles for one grid");
  if (M == 0) return SP_OK;
  if (!x || !w || !dst) return fail(SP_ERR_NULL, "x, w and dst must be non-NULL");
  if (fp8 && (!x_scale || !w_scale)) return fail(SP_ERR_NULL, "x_scale and w_scale must be non-NULL");
  if (misaligned(x) || misaligned(w)) return fail(SP_ERR_ALIGN, "x and w must be 16-byte aligned");
  if (fp8 && (misaligned(x_scale, 4) || misaligned(w_scale, 4)))
    return fail(SP_ERR_ALIGN, "x_scale and w_scale must be 4-byte aligned");
  const size_t e = p->out_dtype == SP_F32 ? 4 : 2;
  const size_t slot_n = static_cast<size_t>(S) * N * e;  // bytes this rank writes per destination
  const size_t ie = fp8 ? 1 : 2;
  const size_t x_n = static_cast<size_t>(M) * K * ie, w_n = static_cast<size_t>(N) * K * ie;
  const size_t xs_n = fp8 ? static_cast<size_t>(p->x_scale_rows) * 4 : 0;
  const size_t ws_n = fp8 ? static_cast<size_t>(p->w_scale_rows) * 4 : 0;
  MArgs ma;
  memset(&ma, 0, sizeof ma);
  for (int r = 0; r < tp; ++r) {
    if (!dst[r]) return fail(SP_ERR_NULL, "dst[%d] is NULL", r);
    if (misaligned(dst[r])) return fail(SP_ERR_ALIGN, "dst[%d] is not 16-byte aligned", r);
    const char* slot = static_cast<const char*>(dst[r]) + static_cast<size_t>(p->rank) * slot_n;
    if (overlap(slot, slot_n, x, x_n) || overlap(slot, slot_n, w, w_n) ||
        overlap(slot, slot_n, x_scale, xs_n) || overlap(slot, slot_n, w_scale, ws_n))
      return fail(SP_ERR_SHAPE, "dst[%d] slot %d overlaps an input", r, p->rank);
    for (int r2 = 0; r2 < r; ++r2) {
      const char* other = static_cast<const char*>(dst[r2]) + static_cast<size_t>(p->rank) * slot_n;
      if (overlap(slot, slot_n, other, slot_n))
        return fail(SP_ERR_SHAPE, "dst[%d] and dst[%d] slots overlap", r, r2);
    }
    ma.dst[r] = static_cast<char*>(dst[r]);
  }
  ma.x = static_cast<const char*>(x);
  ma.w = static_cast<const char*>(w);
  ma.x_scale = x_scale;
  ma.w_scale = w_scale;
  ma.x_scale_rows = static_cast<int32_t>(p->x_scale_rows);
  ma.w_scale_rows = static_cast<int32_t>(p->w_scale_rows);
  ma.S = S;
  ma.slot = static_cast<int64_t>(p->rank) * S;
  ma.M = static_cast<int32_t>(M);
  ma.N = static_cast<int32_t>(N);
  ma.K = static_cast<int32_t>(K);
  ma.tiles_m = static_cast<int32_t>((M + kBM - 1) / kBM);
  ma.tiles_n = static_cast<int32_t>((N + kBN - 1) / kBN);
  void* args[] = {&ma};
  const bool f32 = p->out_dtype == SP_F32;
  const void* fn = fp8 ? (f32 ? reinterpret_cast<const void*>(&matmul_scatter_kernel<SP_F32, SP_FP8_E4M3>)
                              : reinterpret_cast<const void*>(&matmul_scatter_kernel<SP_BF16, SP_FP8_E4M3>))
                       : (f32 ? reinterpret_cast<const void*>(&matmul_scatter_kernel<SP_F32, SP_BF16>)
                              : reinterpret_cast<const void*>(&matmul_scatter_kernel<SP_BF16, SP_BF16>));
  hipError_t err = hipLaunchKernel(fn, dim3(static_cast<unsigned>(tiles)), dim3(kThreads), args, 0,
                                   static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(SP_ERR_HIP, "matmul launch failed: %s", hipGetErrorString(err));
  return SP_OK;
}

}  // namespace

extern "C" {

int sp_matmul_scatter(const sp_matmul_problem* p, const void* x, const void* w, void* const* dst,
                      void* stream) {
  if (!p) return fail(SP_ERR_NULL, "matmul descriptor is NULL");
  if (p->in_dtype != SP_BF16) return fail(SP_ERR_DTYPE, "in_dtype=%d: sp_matmul_scatter takes SP_BF16", p->in_dtype);
  return launch_matmul(p, x, nullptr, w, nullptr, dst, stream);
}

int sp_scaled_matmul_scatter(const sp_matmul_problem* p, const void* x, const float* x_scale,
                             const void* w, const float* w_scale, void* const* dst, void* stream) {
  if (!p) return fail(SP_ERR_NULL, "matmul descriptor is NULL");
  if (p->in_dtype != SP_FP8_E4M3)
    return fail(SP_ERR_DTYPE, "in_dtype=%d: sp_scaled_matmul_scatter takes SP_FP8_E4M3", p->in_dtype);
  return launch_matmul(p, x, x_scale, w, w_scale, dst, stream);
}

}  // extern "C"
