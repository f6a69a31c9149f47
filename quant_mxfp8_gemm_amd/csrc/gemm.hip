// gemm.hip - MXFP8 block-scaled GEMM with BF16 output on gfx950 scaled MFMA.
//
//   C[m,n] = BF16( sum_kb 2^(sa[m,kb]-127) 2^(sb[n,kb]-127) sum_{i<32} A[m,32kb+i] B[n,32kb+i] )
//
// The per-rank GEMM of the o_proj / down_proj GEMM-RS path (vLLM PR #64659, "GEMM-RS
// microbenchmark", N = 6144, K = 2048 / 3072), with the output written in M-row chunks that
// match one rank's reduce-scatter shard ("Overview", "Details").
//
// Design (CDNA4):
//  * Persistent grid: one workgroup per CU walks the output tiles in dispatch order.
//    Tile order: chunk by chunk from first_chunk; inside a chunk every XCD (workgroups are
//    placed round-robin over the 8 XCDs) gets a contiguous run of tiles, grouped GM tile-rows
//    tall, so the 32 tiles an XCD works on at once share A and B panels in its L2.
//  * Large problems use a 256 x 256 output tile split over 8 waves as 4 x 2; each wave owns
//    64 x 128, i.e. 2 x 4 blocks of V_MFMA_SCALE_F32_32X32X64_F8F6F4 accumulated in fp32.
//    Two waves share each SIMD, so one issues MFMAs while the other waits on LDS. Smaller
//    tiles (256 x 192, 192 x 192 and 96 x 192 on 6 waves, 128 x 192, 128 x 128, 64 x 128,
//    32 x 128, with two to four LDS stages) serve problems with fewer rows per chunk; the tile is
//    the one with the shortest estimated makespan (rounds of workgroups over the CUs times the
//    measured time of its K step).
//  * With swizzled, 16-byte aligned scales the 256 x 256 tile runs a split ring: A in two
//    stage buffers and B in three (B fetched two steps ahead, all 160 KiB of LDS), the scales
//    of a wave's rows loaded one step ahead into registers with one 8-byte and one 16-byte
//    load (rows r, r+32, r+64, r+96 of a swizzled 128-row group are adjacent). With BF16
//    output in whole 16-byte segments it, and the 256 x 192 tile, run as two wave groups that
//    take turns on each SIMD's matrix pipe (one issues a half step's MFMAs from registers while
//    the other reads its next fragments from LDS and issues the loads), with a barrier between
//    turns (gemm_pingpong_bf16_kernel, which also serves the fused gate_up epilogue on 256 x 256
//    tiles). Otherwise (unaligned BF16 output, a single 128-K step) its A refill (and the
//    refills of the staged tiles of up to 128 rows) is issued between the two 64-K halves of a
//    step and its B refill after the step's MFMAs, so the step's first fragment reads and MFMAs
//    follow the barrier at once. With at most 32 rows in one chunk (decode) the BF16 GEMM uses one-wave 32 x 32 tiles whose fragments and scales go straight from memory
//    into registers, eight K steps ahead, with no LDS stages or barriers. Every other case uses
//    NS-stage buffers holding A, B and the scale dwords together. All give the same bits:
//    every configuration sums the same MFMA partials in the same order.
//  * The instruction applies the UE8M0 block scales itself. Operand layout (32 rows x 64 K):
//    lane l holds row l%32; with g = l/32, its bytes 0..15 are K 16g..16g+15 and bytes 16..31
//    are K 32+16g..32+16g+15. The scale of (row r, 32-block b) comes from lane r + 32b, byte
//    selected by OPSEL. Result lane l, register v: column l%32, row 8(v/4) + 4(l/32) + v%4.
//    B (output columns n) is fed as the first operand and A as the second, so each lane
//    holds runs of 4 consecutive n of one output row m.
//  * K advances 128 bytes per stage (one full 128-byte line per row). The stages of A, B and
//    their scale dwords live in LDS and are filled straight from memory by LDS-DMA loads:
//    buffer_load_dwordx4 ... lds for A and B (a 32-bit row offset per lane, the stage's K
//    offset in a scalar register), global_load_lds_dword for the staged scales. Each load
//    instruction moves 8 whole rows (8 lanes per 128-byte line). A row of a stage is 8
//    chunks of 16 bytes; chunk c of row r sits in slot c ^ ((r ^ (r >> 3)) & 7), so the rows
//    read by one ds_read_b128 spread over all banks. The 4 scale bytes of a row for one
//    stage are one aligned dword in both scale layouts.
//  * Epilogue: the tile is converted to BF16 into LDS (over the stage buffers, rows padded by
//    16 bytes) and written back with 16-byte streaming stores, every row a run of full lines.
//    The two-group BF16 kernel on 256 x 256 tiles instead has the next tile's first loads in
//    flight (issued by the last K steps when the number of K steps is even) while it writes the
//    tile out in four 32 KiB quarters through the two ring slots those loads leave free, and
//    lets the stores drain under the next tile's first step: all 256 workgroups finish their
//    tiles together, and their stores alone exceed what HBM takes in that time.
//  * A second epilogue serves the fused dense GEMM1 (gate_up projection, SiLU(gate) * up,
//    MXFP8 quantisation; vLLM PR #64659 "Details", PR #64111 "Claims"): a tile's columns are
//    half gate and half up for the same output columns, the fp32 accumulators meet in LDS and
//    each thread turns one (row, 32-block) into E4M3 codes and a UE8M0 scale.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mxfp8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 128;  // K bytes per stage
constexpr int GM = 4;    // tile-rows per group

template <int BM_, int BN_, int WMW, int WNW, int NS_, bool SPLIT_ = false, bool DIRECT_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, NS = NS_;
  // SPLIT: A in a ring of two stage buffers and B in a ring of three (B is fetched two steps
  // ahead), the scales in registers; NS is not used
  static constexpr bool SPLIT = SPLIT_;
  // DIRECT: no LDS stages; each wave loads its own MFMA fragments and scales from global
  // memory into registers, NS steps ahead (LDS only stages the output tile)
  static constexpr bool DIRECT = DIRECT_;
  static constexpr int NW = WMW * WNW, NT = NW * 64;
  static constexpr int WTM = BM / WMW, WTN = BN / WNW;  // wave sub-tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;    // MFMA blocks per wave
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, SC_BYTES = (BM + BN) * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
  static constexpr int DA = A_BYTES / 1024 / NW;  // 1 KiB data loads per wave per stage
  static constexpr int DB = B_BYTES / 1024 / NW;
  static constexpr int SROWS = (BM + BN) / NW;    // scale rows (one dword each) per wave per stage
  static constexpr int DS = (SROWS + 63) / 64;    // scale loads per wave per stage
  static constexpr int LOADS = DA + DB + DS;      // LDS-DMA instructions per wave per stage
  static constexpr int C_STRIDE = BN * 2 + 16;    // bytes per staged output row
  static constexpr int RING_BYTES = SPLIT ? 2 * A_BYTES + 3 * B_BYTES : DIRECT ? 0 : NS * STAGE;
  static constexpr int LDS_BYTES = RING_BYTES > BM * C_STRIDE ? RING_BYTES : BM * C_STRIDE;
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(DA * NW * 1024 == A_BYTES && DB * NW * 1024 == B_BYTES, "data split");
  static_assert(SROWS * NW == BM + BN && (SROWS % 64 == 0 || SROWS < 64), "scale split");
  static_assert(NS >= 2 && LDS_BYTES <= 160 * 1024, "stages");
  static_assert((BM * BN / 8) % NT == 0, "epilogue rows");
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Workgroup barrier without a memory fence. LDS-DMA completions are waited for explicitly
// (vmcnt) before it, and each wave drains its own LDS accesses (lgkmcnt) so no buffer is
// refilled or reread under a pending access; the epilogue's global stores need not drain.
__device__ __forceinline__ void block_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// An 8-byte LDS store that the compiler does not see as one. The compiler cannot tell which LDS
// bytes an LDS-DMA load in flight writes, so it makes a store to LDS wait for all of them; this
// store is for LDS that the caller knows no load in flight targets. It completes in order with
// the wave's other LDS accesses (a later wait on lgkmcnt covers it).
__device__ __forceinline__ void lds_store_b64_unordered(uint8_t* p, u32x2 v) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)p;
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}

// Wait until at most N of this wave's vector memory operations are outstanding. They
// complete in issue order, so this means every load issued before the last N has landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Byte offset, inside one stage's A or B region, of logical 16-byte chunk c of row r.
__device__ __forceinline__ int lds_off(int r, int c) { return (r * 8 + (c ^ swz(r))) * 16; }

#if defined(__HIP_DEVICE_COMPILE__)
// Raw buffer resource over [p, p + bytes) (gfx9 descriptor word 3); loads past the end read 0.
// Device pass only: the host pass of this toolchain drops the kernel stubs when the
// resource type appears in a kernel body, so the buffer code is compiled for the GPU alone.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
#endif

template <int SEL>
__device__ __forceinline__ v16f mfma(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, sa, SEL, sb);
}

// Wait as wait_vm<N>, and tell the compiler that the two scale vectors are only final after
// it: they are the destinations of loads the compiler does not track (split ring below).
template <int N>
__device__ __forceinline__ void wait_vm_regs(u32x2& a, u32x4& b) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}

// Offset of the 4-byte scale group (row r, 128-K step 0) in the given layout; nblk4 = K/128.
template <int LAYOUT>
__device__ __forceinline__ uint32_t scale_base(uint32_t r, uint32_t nblk4) {
  if (LAYOUT == 0) return r * nblk4 * 4;
  return (r >> 7) * nblk4 * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4;
}
// Distance between consecutive 128-K steps of one row's scale dwords.
template <int LAYOUT>
constexpr uint32_t scale_step() { return LAYOUT == 0 ? 4u : 512u; }

// Fragment offsets inside a stage: the swizzle of row r + 32 t is that of row r with bit 2
// flipped when t is odd (which swaps the two 64-K halves of the row), so four per-lane offsets
// per operand, relative to the wave's first row, address every fragment read; the rest is a
// constant (t * 32 rows).
template <class T>
__device__ __forceinline__ void frag_offsets(int wm, int wn, int l32, int g, int (&oa)[2][2], int (&ob)[2][2]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      oa[kk][h] = lds_off(wm * T::WTM + l32, 4 * kk + 2 * h + g) - wm * T::WTM * 128;
      ob[kk][h] = lds_off(wn * T::WTN + l32, 4 * kk + 2 * h + g) - wn * T::WTN * 128;
    }
}

// One 128-K step of a wave's TM x TN blocks from LDS: two 64-K halves, each one scaled MFMA per
// (B block, A block); between_halves runs after the first half's MFMAs are issued.
template <class T, class F>
__device__ __forceinline__ void lds_mma_step(v16f (&acc)[T::TN][T::TM], const uint8_t* a_lds, const uint8_t* b_lds,
                                             int wm, int wn, const int (&oa)[2][2], const int (&ob)[2][2],
                                             const uint32_t* as_sel, const uint32_t* bs_sel, F&& between_halves) {
  const uint8_t* const a_w = a_lds + wm * T::WTM * 128;
  const uint8_t* const b_w = b_lds + wn * T::WTN * 128;
  // the compiler's predefined LDS-read / MFMA interleave (strategy 0) for this region
  __builtin_amdgcn_iglp_opt(0);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    v8i af[T::TM], bf[T::TN];
#pragma unroll
    for (int t = 0; t < T::TM; ++t) {
      const int kk = ks ^ (t & 1);
      const v4i lo = *(const v4i*)(a_w + oa[kk][0] + t * 32 * 128);
      const v4i hi = *(const v4i*)(a_w + oa[kk][1] + t * 32 * 128);
      af[t] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int t = 0; t < T::TN; ++t) {
      const int kk = ks ^ (t & 1);
      const v4i lo = *(const v4i*)(b_w + ob[kk][0] + t * 32 * 128);
      const v4i hi = *(const v4i*)(b_w + ob[kk][1] + t * 32 * 128);
      bf[t] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int x = 0; x < T::TN; ++x)
#pragma unroll
      for (int y = 0; y < T::TM; ++y) {
        if (ks == 0)
          acc[x][y] = mfma<0>(bf[x], af[y], acc[x][y], (int)bs_sel[x], (int)as_sel[y]);
        else
          acc[x][y] = mfma<2>(bf[x], af[y], acc[x][y], (int)bs_sel[x], (int)as_sel[y]);
      }
    if (ks == 0) between_halves();
  }
}

// Outputs of the fused dense GEMM1 epilogue (EPI_SWIGLU): B holds 2*inter rows, gate then up.
struct SwiGluOut {
  uint8_t* q;      // [M, inter] E4M3
  uint8_t* s_lin;  // [M, inter/32] or null
  uint8_t* s_swz;  // swizzled [M, inter/32] or null
  int inter;
};

enum { EPI_BF16 = 0, EPI_SWIGLU = 1 };

// Fused dense GEMM1 epilogue of one tile (EPI_SWIGLU) from the accumulators of the wave at
// (wm, wn): fp32 gate and up staged in LDS a band of rows at a time, then one (row, 32-block of j)
// per thread: y = SiLU(g) * u, UE8M0 scale from amax, E4M3 codes. The caller makes sure nothing
// else reads or writes the tile's LDS meanwhile.
template <class T>
__device__ __forceinline__ void swiglu_epilogue(uint8_t* smem, const v16f (&acc)[T::TN][T::TM], int wm, int wn,
                                                int l32, int g, int tid, int m0, int m_end, int n0,
                                                const SwiGluOut& sg) {
  constexpr int BM = T::BM, BN = T::BN, HB = BN / 2;
  // ---- fused epilogue: fp32 gate and up staged in LDS a band of rows at a time, then one
  // (row, 32-block of j) per thread: y = SiLU(g) * u, UE8M0 scale from amax, E4M3 codes
  // Bytes per staged row (gate floats, then up floats). A staged column c sits at
  // c ^ 16 where bit 6 of c is set: the readers below take 16 rows x 4 blocks of 32 columns
  // at a time, and without it blocks b and b + 2 of a row would share their banks.
  constexpr int SROW = BN * 4 + 16;
  constexpr int FIT = T::LDS_BYTES / SROW;
  // rows per band: the whole tile, else half or a quarter of it, whatever fits
  constexpr int PR = FIT >= BM ? BM : FIT >= BM / 2 ? BM / 2 : BM / 4;
  static_assert(PR >= 32 && BM % PR == 0 && T::WTM % 32 == 0, "fused epilogue bands");
  constexpr int BPR = HB / 32;  // 32-blocks of j per tile row
  const int nblk = sg.inter / 32;
  const int64_t col_tiles = (nblk + 3) / 4;
#pragma unroll
  for (int p0 = 0; p0 < BM; p0 += PR) {
    block_barrier();  // the stages (or the previous band) are no longer read
#pragma unroll
    for (int y = 0; y < T::TM; ++y) {
      const int rb = wm * T::WTM + y * 32;
      if (rb < p0 || rb >= p0 + PR) continue;
      const int r = rb - p0 + l32;
#pragma unroll
      for (int x = 0; x < T::TN; ++x)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * T::WTN + x * 32 + 8 * q + 4 * g;
          *(float4*)(smem + r * SROW + (c ^ (((c >> 6) & 1) << 4)) * 4) =
              make_float4(acc[x][y][4 * q + 0], acc[x][y][4 * q + 1], acc[x][y][4 * q + 2], acc[x][y][4 * q + 3]);
        }
    }
    block_barrier();
    for (int it = tid; it < PR * BPR; it += T::NT) {
      const int r = it / BPR, b = it % BPR;
      const int m = m0 + p0 + r;
      const int j = n0 + 32 * b;
      if (m >= m_end || j >= sg.inter) continue;
      const float* gp = (const float*)(smem + r * SROW) + 32 * b;
      const float* up = gp + HB;
      const int xg = ((32 * b) & 64) >> 2, xu = ((32 * b + HB) & 64) >> 2;  // the column swizzle
      float yv[32];
      uint32_t amax = 0;
#pragma unroll
      for (int e = 0; e < 32; e += 4) {
        const float4 g4 = *(const float4*)(gp + (e ^ xg));
        const float4 u4 = *(const float4*)(up + (e ^ xu));
        const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
        const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float v = gg[t] / (1.0f + expf(-gg[t])) * uu[t];
          yv[e + t] = v;
          amax = max(amax, __float_as_uint(v) & 0x7FFFFFFFu);
        }
      }
      const uint32_t code = ue8m0_from_amax_f32_bits(amax);
      const float inv = inv_scale_from_ue8m0(code);
      uint32_t w[8];
#pragma unroll
      for (int t = 0; t < 8; ++t)
        w[t] = cvt_e4m3x4(yv[4 * t] * inv, yv[4 * t + 1] * inv, yv[4 * t + 2] * inv, yv[4 * t + 3] * inv);
      uint8_t* qd = sg.q + (int64_t)m * sg.inter + j;
      __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]}, (u32x4*)qd);
      __builtin_nontemporal_store((u32x4){w[4], w[5], w[6], w[7]}, (u32x4*)(qd + 16));
      if (sg.s_lin) sg.s_lin[(int64_t)m * nblk + j / 32] = (uint8_t)code;
      if (sg.s_swz) sg.s_swz[swizzled_offset(m, j / 32, col_tiles)] = (uint8_t)code;
    }
  }
}

template <class T, int A_LAYOUT, int B_LAYOUT, int EPI>
__global__ __launch_bounds__(T::NT, 1) void gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int ldc, int num_chunks,
    int first_chunk, int* __restrict__ chunk_done, int wide_store, SwiGluOut sg) {
  constexpr int BM = T::BM, BN = T::BN, NS = T::NS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (an SGPR): the LDS-DMA destinations and M0 are formed with scalar instructions
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (BN / T::WTN), wn = wave % (BN / T::WTN);
  const int l32 = lane & 31, g = lane >> 5;

  const int chunk_rows = M / num_chunks;
  // EPI_SWIGLU: a tile's BN columns are BN/2 gate columns j0.. and the BN/2 up columns of the
  // same j, so SiLU(gate) * up of an output element is formed inside one tile
  constexpr int HB = BN / 2;
  const int tiles_n = EPI == EPI_SWIGLU ? (sg.inter + HB - 1) / HB : (N + BN - 1) / BN;
  const int tiles_mc = (chunk_rows + BM - 1) / BM;
  const int tpc = tiles_mc * tiles_n;
  const int total = tpc * num_chunks;
  const int KT = K / BK;
  const uint32_t nblk4 = (uint32_t)K / 128;

  for (int bid = blockIdx.x; bid < total; bid += gridDim.x) {
    // ---- tile coordinates
    const int ci = bid / tpc;
    const int j = bid - ci * tpc;
    const int chunk = (first_chunk + ci) % num_chunks;
    const int lj = (tpc % 8 == 0) ? (j % 8) * (tpc / 8) + j / 8 : j;
    const int group = lj / (GM * tiles_n);
    const int first_tm = group * GM;
    const int gsz = min(tiles_mc - first_tm, GM);
    const int tm_idx = first_tm + (lj % (GM * tiles_n)) % gsz;
    const int tn_idx = (lj % (GM * tiles_n)) / gsz;
    const int chunk_m0 = chunk * chunk_rows;
    const int m0 = chunk_m0 + tm_idx * BM;
    const int m_end = min(m0 + BM, chunk_m0 + chunk_rows);
    const int n0 = tn_idx * (EPI == EPI_SWIGLU ? HB : BN);  // first output column (j0 for EPI_SWIGLU)
    // B row that feeds tile column r (clamped into the operand; surplus columns are not stored)
    auto b_row = [&](int r) -> uint32_t {
      if (EPI == EPI_SWIGLU)
        return r < HB ? (uint32_t)min(n0 + r, sg.inter - 1) : (uint32_t)(sg.inter + min(n0 + r - HB, sg.inter - 1));
      return (uint32_t)min(n0 + r, N - 1);
    };

    // ---- per-lane LDS-DMA sources (rows clamped into the operand; surplus rows are not stored)
    uint32_t a_off[T::DA], b_off[T::DB], s_off[T::DS];
    const uint8_t* s_src[T::DS];
    uint32_t s_step[T::DS];
#pragma unroll
    for (int i = 0; i < T::DA; ++i) {
      const int s = (wave * T::DA + i) * 64 + lane;
      const int r = s >> 3;
      a_off[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + (((s & 7) ^ swz(r)) * 16);
    }
#pragma unroll
    for (int i = 0; i < T::DB; ++i) {
      const int s = (wave * T::DB + i) * 64 + lane;
      const int r = s >> 3;
      b_off[i] = b_row(r) * (uint32_t)K + (((s & 7) ^ swz(r)) * 16);
    }
#pragma unroll
    for (int i = 0; i < T::DS; ++i) {
      // A rows first, then B rows; with fewer than 64 rows per wave the upper lanes repeat
      // the wave's last row (same source, same LDS slot contents).
      const int row = wave * T::SROWS + i * 64 + min(lane, T::SROWS - 1);
      if (row < BM) {
        s_src[i] = As;
        s_off[i] = scale_base<A_LAYOUT>((uint32_t)min(m0 + row, M - 1), nblk4);
        s_step[i] = scale_step<A_LAYOUT>();
      } else {
        s_src[i] = Bs;
        s_off[i] = scale_base<B_LAYOUT>(b_row(row - BM), nblk4);
        s_step[i] = scale_step<B_LAYOUT>();
      }
    }

    auto issue = [&](int kt, int buf) {
      uint8_t* st = smem + buf * T::STAGE;
      const uint32_t k0 = (uint32_t)kt * BK;
#if defined(__HIP_DEVICE_COMPILE__)
      // A and B through buffer resources: per-lane 32-bit row offsets, the K offset of the
      // stage in a scalar register
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * (uint32_t)K);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (uint32_t)N * (uint32_t)K);
#pragma unroll
      for (int i = 0; i < T::DA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (wave * T::DA + i) * 1024), 16, a_off[i], k0, 0, 0);
#pragma unroll
      for (int i = 0; i < T::DB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + T::A_BYTES + (wave * T::DB + i) * 1024), 16,
                                                 b_off[i], k0, 0, 0);
#endif
#pragma unroll
      for (int i = 0; i < T::DS; ++i) {
        if (T::SROWS >= 64) {
          __builtin_amdgcn_global_load_lds((const void*)(s_src[i] + s_off[i] + (uint32_t)kt * s_step[i]),
                                           (lds_void*)(st + T::A_BYTES + T::B_BYTES + (wave * T::SROWS + i * 64) * 4),
                                           4, 0, 0);
        } else {
          // fewer rows than lanes: the surplus lanes write past this wave's slice, so they
          // are masked off (the instruction still counts once in vmcnt for the wave)
          if (lane < T::SROWS)
            __builtin_amdgcn_global_load_lds((const void*)(s_src[i] + s_off[i] + (uint32_t)kt * s_step[i]),
                                             (lds_void*)(st + T::A_BYTES + T::B_BYTES + wave * T::SROWS * 4),
                                             4, 0, 0);
        }
      }
    };

    v16f acc[T::TN][T::TM];
#pragma unroll
    for (int x = 0; x < T::TN; ++x)
#pragma unroll
      for (int y = 0; y < T::TM; ++y)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.f;

    // fragment offsets inside a stage (frag_offsets)
    int oa[2][2], ob[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        oa[kk][h] = lds_off(wm * T::WTM + l32, 4 * kk + 2 * h + g) - wm * T::WTM * 128;
        ob[kk][h] = lds_off(wn * T::WTN + l32, 4 * kk + 2 * h + g) - wn * T::WTN * 128;
      }
    auto mma_step = [&](const uint8_t* a_lds, const uint8_t* b_lds, const uint32_t* as_sel,
                        const uint32_t* bs_sel, auto&& between_halves) {
      lds_mma_step<T>(acc, a_lds, b_lds, wm, wn, oa, ob, as_sel, bs_sel, between_halves);
    };

    if constexpr (T::SPLIT) {
      static_assert(A_LAYOUT == 1 && B_LAYOUT == 1 && T::TM == 2 && T::TN == 4 && T::WTM == 64 && T::WTN == 128,
                    "split ring: swizzled scales, 64 x 128 wave tiles");
#if defined(__HIP_DEVICE_COMPILE__)
      // In the swizzled layout rows r, r + 32, r + 64, r + 96 of a 128-row group keep their
      // 4-byte scale groups side by side. A wave's A rows are r0 + l32 and r0 + 32 + l32 with
      // r0 a multiple of 64 (chunks start on 64-row boundaries), its B rows b0 + l32 + 32t with
      // b0 a multiple of 128 (EPI_SWIGLU: the wave's 128 gate or up rows, inter a multiple of
      // 128): one 8-byte and one 16-byte load per lane and step. Rows past the operand read
      // the zero padding of the 128-row group or, beyond the buffer, 0 (not stored either way).
      uint8_t* const a_ring = smem;
      uint8_t* const b_ring = smem + 2 * T::A_BYTES;
      const uint32_t sa_off = scale_base<1>((uint32_t)(m0 + wm * T::WTM + l32), nblk4);
      const int b0 = EPI == EPI_SWIGLU ? (wn == 0 ? n0 : sg.inter + n0) : n0 + wn * T::WTN;
      const uint32_t sb_off = scale_base<1>((uint32_t)(b0 + l32), nblk4);
      const uint32_t sa_bytes = (uint32_t)((M + 127) / 128 * 128) * nblk4 * 4;
      const uint32_t sb_bytes = (uint32_t)((N + 127) / 128 * 128) * nblk4 * 4;
      const __amdgpu_buffer_rsrc_t rsa = make_rsrc(As, sa_bytes), rsb = make_rsrc(Bs, sb_bytes);
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * (uint32_t)K);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (uint32_t)N * (uint32_t)K);
      auto issue_a = [&](int kt) {
        uint8_t* st = a_ring + (kt & 1) * T::A_BYTES;
#pragma unroll
        for (int i = 0; i < T::DA; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (wave * T::DA + i) * 1024), 16, a_off[i],
                                                   (uint32_t)kt * BK, 0, 0);
      };
      auto issue_b = [&](int kt, int slot) {
        uint8_t* st = b_ring + slot * T::B_BYTES;
#pragma unroll
        for (int i = 0; i < T::DB; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + (wave * T::DB + i) * 1024), 16, b_off[i],
                                                   (uint32_t)kt * BK, 0, 0);
      };
      auto load_scales = [&](int kt, u32x2& sa, u32x4& sb) {
        const int so = kt * (int)scale_step<1>();
        sa = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsa, sa_off, so, 0));
        sb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsb, sb_off, so, 0));
      };
      // Every load of the steady state is issued unconditionally and the last two steps are
      // peeled: the compiler's own wait before the first use of the scales then counts the
      // same B loads behind them on every path (vmcnt(DB), as the explicit wait), where a
      // conditional issue would make it wait for all loads (vmcnt(0)).
      u32x2 sa;  // scales of the step about to run (loaded one step ahead)
      u32x4 sb;
      block_barrier();  // the previous tile's epilogue is done with LDS
      issue_b(0, 0);
      issue_a(0);
      load_scales(0, sa, sb);
      int bslot = 0;  // B buffer of step kt
      auto step = [&](int kt, bool next_a, bool next_b) {
        block_barrier();
        // this lane's scale bytes: byte 0 -> block g (first 64 K), byte 2 -> block 2+g
        uint32_t as_sel[2], bs_sel[4];
#pragma unroll
        for (int t = 0; t < 2; ++t) as_sel[t] = (sa[t] >> (8 * g)) & 0x00FF00FFu;
#pragma unroll
        for (int t = 0; t < 4; ++t) bs_sel[t] = (sb[t] >> (8 * g)) & 0x00FF00FFu;
        const int refill = bslot == 0 ? 2 : bslot - 1;
        const uint8_t* a_lds = a_ring + (kt & 1) * T::A_BYTES;
        const uint8_t* b_lds = b_ring + bslot * T::B_BYTES;
        bslot = bslot == 2 ? 0 : bslot + 1;
        // refill the A buffer read at step kt - 1 between the two 64-K halves (the first half's
        // fragment reads and MFMAs start right after the barrier), and the B buffer read at step
        // kt - 1 after the step's MFMAs (B is fetched two steps ahead, so it can wait)
        mma_step(a_lds, b_lds, as_sel, bs_sel, [&] {
          if (next_a) {
            issue_a(kt + 1);
            load_scales(kt + 1, sa, sb);
            // keep the scale loads ahead of the B loads: issued behind them they would be among
            // the last DB loads, and the next step's wait would also wait for part of B(kt + 2)
            __builtin_amdgcn_sched_barrier(0);
          }
        });
        if (next_b) issue_b(kt + 2, refill);
      };
      // A(kt), the scales of kt and B(kt) have landed before each step; B(kt + 1) may not have.
      // A single K step has a path of its own, so that the registers of the last step's scales
      // come from one place (a merge would have the compiler copy them, and wait for them,
      // before the step ahead of it is done).
      if (KT == 1) {
        wait_vm<0>();
        step(0, false, false);
      } else {
        issue_b(1, 1);
        for (int kt = 0; kt < KT - 2; ++kt) {
          wait_vm<T::DB>();
          step(kt, true, true);
        }
        wait_vm<T::DB>();
        step(KT - 2, true, false);
        wait_vm<0>();
        step(KT - 1, false, false);
      }
#endif
    } else if constexpr (T::DIRECT) {
      static_assert(T::TM == 1 && T::TN == 1 && EPI == EPI_BF16, "direct loads: one 32 x 32 block per wave");
#if defined(__HIP_DEVICE_COMPILE__)
      // Lane (l32, g) holds, for each 64-K half, the 16 bytes at K 16g and at K 32 + 16g of its
      // A row and of its B row: the operand layout of the scaled MFMA, loaded as the LDS path
      // reads it, so the products and their order are the same. Rows past the operand repeat
      // its last row (their outputs are not stored).
      constexpr int P = T::NS;  // steps in flight
      const uint32_t arow = (uint32_t)min(m0 + wm * T::WTM + l32, M - 1);
      const uint32_t brow = b_row(wn * T::WTN + l32);
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * (uint32_t)K);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (uint32_t)N * (uint32_t)K);
      const uint32_t a_vo = arow * (uint32_t)K + 16 * g, b_vo = brow * (uint32_t)K + 16 * g;
      const uint8_t* const sa_p = As + scale_base<A_LAYOUT>(arow, nblk4);
      const uint8_t* const sb_p = Bs + scale_base<B_LAYOUT>(brow, nblk4);
      v4i fa[P][4], fb[P][4];
      uint32_t fsa[P], fsb[P];
      // every load is issued unconditionally (steps past the end reload the last one), so the
      // compiler's count of loads in flight is the same on every path
      auto load = [&](int kt, int u) {
        kt = min(kt, KT - 1);
        const int k0 = kt * BK;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          fa[u][q] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, a_vo, k0 + 32 * q, 0));
          fb[u][q] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, b_vo, k0 + 32 * q, 0));
        }
        fsa[u] = *(const uint32_t*)(sa_p + (uint32_t)kt * scale_step<A_LAYOUT>());
        fsb[u] = *(const uint32_t*)(sb_p + (uint32_t)kt * scale_step<B_LAYOUT>());
      };
#pragma unroll
      for (int u = 0; u < P; ++u) load(u, u);
      for (int kt0 = 0; kt0 < KT; kt0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
          if (kt0 + u < KT) {
            const int as_sel = (int)((fsa[u] >> (8 * g)) & 0x00FF00FFu);
            const int bs_sel = (int)((fsb[u] >> (8 * g)) & 0x00FF00FFu);
            const v4i* a4 = fa[u];
            const v4i* b4 = fb[u];
            const v8i a0 = {a4[0][0], a4[0][1], a4[0][2], a4[0][3], a4[1][0], a4[1][1], a4[1][2], a4[1][3]};
            const v8i a1 = {a4[2][0], a4[2][1], a4[2][2], a4[2][3], a4[3][0], a4[3][1], a4[3][2], a4[3][3]};
            const v8i b0 = {b4[0][0], b4[0][1], b4[0][2], b4[0][3], b4[1][0], b4[1][1], b4[1][2], b4[1][3]};
            const v8i b1 = {b4[2][0], b4[2][1], b4[2][2], b4[2][3], b4[3][0], b4[3][1], b4[3][2], b4[3][3]};
            acc[0][0] = mfma<0>(b0, a0, acc[0][0], bs_sel, as_sel);
            acc[0][0] = mfma<2>(b1, a1, acc[0][0], bs_sel, as_sel);
          }
          load(kt0 + u + P, u);
        }
      }
#endif
    } else {
      block_barrier();  // the previous tile's epilogue is done with LDS
#pragma unroll
      for (int s = 0; s < NS - 1; ++s)
        if (s < KT) issue(s, s);
      int buf = 0;                // buffer of stage kt
      int fill = NS - 1;          // buffer that stage kt + NS - 1 goes to
      for (int kt = 0; kt < KT; ++kt) {
        // stage kt has landed in LDS for every wave; up to NS - 2 later stages stay in flight
        if (kt + NS - 2 < KT)
          wait_vm<(NS - 2) * T::LOADS>();
        else
          wait_vm<0>();
        block_barrier();
        // refill the buffer read at step kt - 1: tiles of up to 128 rows issue the refill between
        // the two 64-K halves (their first reads and MFMAs start at once; measured 2-3.5% faster),
        // larger tiles right after the barrier (measured 1.5-4.5% faster that way)
        constexpr bool kRefillMid = BM <= 128;
        const int fill_now = fill;
        if (!kRefillMid && kt + NS - 1 < KT) issue(kt + NS - 1, fill_now);
        fill = fill + 1 == NS ? 0 : fill + 1;

        const uint8_t* st = smem + buf * T::STAGE;
        buf = buf + 1 == NS ? 0 : buf + 1;
        const uint8_t* a_lds = st;
        const uint8_t* b_lds = st + T::A_BYTES;
        const uint32_t* sc = (const uint32_t*)(st + T::A_BYTES + T::B_BYTES);
        // this lane's scale bytes: byte 0 -> block g (first 64 K), byte 2 -> block 2+g (second 64 K)
        uint32_t as_sel[T::TM], bs_sel[T::TN];
#pragma unroll
        for (int t = 0; t < T::TM; ++t) as_sel[t] = (sc[wm * T::WTM + t * 32 + l32] >> (8 * g)) & 0x00FF00FFu;
#pragma unroll
        for (int t = 0; t < T::TN; ++t) bs_sel[t] = (sc[BM + wn * T::WTN + t * 32 + l32] >> (8 * g)) & 0x00FF00FFu;
        mma_step(a_lds, b_lds, as_sel, bs_sel, [&] {
          if (kRefillMid && kt + NS - 1 < KT) issue(kt + NS - 1, fill_now);
        });
      }
    }  // main loop

    if constexpr (EPI == EPI_SWIGLU) {
      swiglu_epilogue<T>(smem, acc, wm, wn, l32, g, tid, m0, m_end, n0, sg);
      continue;  // next tile (the fused output has no chunk counters)
    }

    // ---- epilogue: BF16 tile staged in LDS, then full-line 16-byte stores. A staged row is
    // 16 bytes longer than the tile row, so rows r and r + 8 (and r + 16) start in the same
    // bank; each 8-byte write fills one half of a 16-byte group, and rows where bit 3 xor bit 4
    // of r is set swap the halves of every group, so that the 32 rows of one write hit
    // distinct banks (the readers swap them back).
    block_barrier();  // every wave is done reading the last stage
#pragma unroll
    for (int x = 0; x < T::TN; ++x) {
#pragma unroll
      for (int y = 0; y < T::TM; ++y) {
        const int r = wm * T::WTM + y * 32 + l32;
        const int gs = g ^ (((r >> 3) ^ (r >> 4)) & 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * T::WTN + x * 32 + 8 * q + 4 * gs;
          const uint32_t lo = pack_bf16x2(acc[x][y][4 * q + 0], acc[x][y][4 * q + 1]);
          const uint32_t hi = pack_bf16x2(acc[x][y][4 * q + 2], acc[x][y][4 * q + 3]);
          *(uint2*)(smem + r * T::C_STRIDE + c * 2) = make_uint2(lo, hi);
        }
      }
    }
    block_barrier();
    constexpr int SEGS = BN / 8;  // 16-byte segments per row
#pragma unroll 4
    for (int p = tid; p < BM * SEGS; p += T::NT) {
      const int r = p / SEGS;
      const int c8 = (p % SEGS) * 8;
      const int m = m0 + r;
      const int n = n0 + c8;
      if (m >= m_end || n >= N) continue;
      uint4 v = *(const uint4*)(smem + r * T::C_STRIDE + c8 * 2);
      if (((r >> 3) ^ (r >> 4)) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
      uint16_t* dst = C + (int64_t)m * ldc + n;
      if (n + 8 <= N) {
        if (wide_store) {
          __builtin_nontemporal_store(*(const u32x4*)&v, (u32x4*)dst);
        } else {
          *(uint2*)dst = make_uint2(v.x, v.y);
          *(uint2*)(dst + 4) = make_uint2(v.z, v.w);
        }
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int e = 0; e < N - n; ++e) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }

    if (chunk_done != nullptr) {
      __threadfence();  // this thread's C stores are visible device-wide
      __syncthreads();
      if (tid == 0) atomicAdd(chunk_done + chunk, 1);
    }
  }
}

// GEMM on 256 x 256 or 256 x 192 tiles whose eight waves take turns on the matrix pipes, with
// BF16 output or the fused gate_up epilogue. Waves 0-3 (tile rows 0-127) and waves 4-7 (rows 128-255) put one wave of each group on
// every SIMD. Each wave alternates a memory phase (the LDS fragment reads of one 64-K half step
// into registers, then its share of the loads) and a compute phase (the half step's scaled
// MFMAs from those registers), with a workgroup barrier after every phase; the second group
// starts one phase late, so that on each SIMD one wave issues MFMAs while the other reads its
// next fragments. B is in a ring of three LDS slots (fetched two steps ahead) and A in two (one
// step ahead), the scales in registers one step ahead. Each group loads the A rows that only it
// reads, so the refill of an A slot waits only for that group's last reads of it.
//  * A memory phase issues no vector ALU work: an MFMA waiting for the matrix pipe holds the
//    SIMD's vector issue, so ALU work in one wave's memory phase would wait on the other wave's
//    MFMAs. The LDS addresses are per-lane bases fixed for the tile plus instruction offsets;
//    the loop is unrolled over six steps (two A slots, three B slots, two scale register sets)
//    so that every slot offset is a constant.
//  * A load instruction can take hundreds of cycles to issue when the memory pipeline is busy,
//    so the loads are issued in the memory phases, after the fragment reads.
//  * Per step and wave the loads leave in one order (A scales of step s + 1, A(s + 1), then
//    B(s + 2), B scales of step s + 1), so that two fixed counts wait for B(s + 1) before the
//    last barrier that precedes its first read and for A(s + 1) before the group's own first
//    read. Loads past the last step go through empty resources (dropped) so that the counts
//    hold on every path.
//  * 256 x 256, BF16: the next tile's B(0), scales, A(0) and B(1) (A slot 0, B slots 0 and 1)
//    are issued by the tile's last two steps when its number of K steps is even (chained),
//    else after its last step; then the tile leaves in four quarters of 128 rows x 128 columns
//    staged alternately in A slot 1 and B slot 2. The C stores are buffer stores over the
//    tile's own rows (elements past the last row or column are dropped), so every wave issues
//    the same 16 stores, and the next tile's first waits let exactly those stay in flight.
//    256 x 192 (two tiles per compute unit at most, for the M = 1536-4096 workloads) and the
//    fused epilogue: the whole tile (fused: fp32 bands of it) is staged once every load has
//    landed, then the next tile's first loads are issued.
template <class T, int CH, int EPI = EPI_BF16>
__global__ __launch_bounds__(T::NT, 1) void gemm_pingpong_bf16_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, uint16_t* __restrict__ C, int M, int N, int K, int ldc, int num_chunks,
    int first_chunk, int* __restrict__ chunk_done, SwiGluOut sg = SwiGluOut{}) {
  constexpr int BM = T::BM, BN = T::BN;
  // EPI_SWIGLU (fused dense GEMM1): a tile's columns are HB gate columns j0.. and the HB up
  // columns of the same j (B rows j0.. and inter + j0..; inter a multiple of HB, checked by the
  // caller), and its epilogue writes E4M3 codes and scales of SiLU(gate) * up
  constexpr int HB = BN / 2;
  static_assert(EPI == EPI_BF16 || CH == 0, "fused epilogue: unchained");
  static_assert(T::SPLIT && BM == 256 && (BN == 256 || BN == 192) && T::TM == 2 && T::NT == 512 &&
                    T::DA == 4 && T::WTM == 64 && T::A_BYTES == 32768 && T::WTN == BN / 2,
                "256-row tiles of 8 waves of 64 x BN/2");
  constexpr int TN = T::TN;
  // overlapped epilogue (quarters through A slot 1 and B slot 2): 256 x 256
  constexpr bool OVL = BN == 256 && EPI == EPI_BF16;
  // B slots at 0, 1 and 2 B_BYTES, A slots after them
  constexpr int B_RING = 0, A_RING = 3 * T::B_BYTES;
  static_assert(A_RING + 2 * T::A_BYTES <= 160 * 1024, "ring");
  // B slot 2 lies beyond the 64 KiB reach of an instruction offset from the slot-0 base
  constexpr bool FAR_B2 = 2 * T::B_BYTES + (TN - 1) * 32 * 128 + 32 * 128 > 65536;
  // B scale loads per step: one 16-byte load. 256 x 256: the wave's four row blocks, one
  // swizzled 128-row group. 256 x 192: the wave's three blocks start at block q of a group and
  // may run into the next one, so lanes 0-31 load the group of the first block and lanes 32-63
  // the group after it, and a lane-half swap gives every lane both (SB_TWO_GROUPS)
  constexpr int NSB = 1;
  constexpr bool SB_TWO_GROUPS = BN == 192;
  constexpr int SBW = SB_TWO_GROUPS ? 4 : TN;  // B scale dwords a lane keeps per step
  constexpr int C_STORES = OVL ? 16 : 0;  // C stores per thread and tile left in flight
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
#if defined(__HIP_DEVICE_COMPILE__)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: tile rows 0-127, 1: rows 128-255
  const int wm = wave / (BN / T::WTN), wn = wave % (BN / T::WTN);
  const int g = lane >> 5;

  const int chunk_rows = M / num_chunks;
  const int tiles_n = EPI == EPI_SWIGLU ? sg.inter / HB : (N + BN - 1) / BN;
  const int tiles_mc = (chunk_rows + BM - 1) / BM;
  const int tpc = tiles_mc * tiles_n;
  const int total = tpc * num_chunks;
  const int KT = K / BK;
  const uint32_t nblk4 = (uint32_t)K / 128;

  const uint32_t sa_bytes = (uint32_t)((M + 127) / 128 * 128) * nblk4 * 4;
  const uint32_t sb_bytes = (uint32_t)((N + 127) / 128 * 128) * nblk4 * 4;
  const uint32_t a_bytes = (uint32_t)M * (uint32_t)K, b_bytes = (uint32_t)N * (uint32_t)K;
  // overlapped epilogue staging: A slot 1 and B slot 2 (the next tile's first loads use the others)
  uint8_t* const stage0 = smem + A_RING + T::A_BYTES;
  uint8_t* const stage1 = smem + B_RING + 2 * T::B_BYTES;

  // ---- per-tile state: output origin and the offsets of its loads
  struct TileState {
    int m0, m_end, n0, chunk;
    uint32_t a_off[T::DA], b_off[T::DB], sa_off, sb_off[NSB];
    int sbq;  // 256 x 192: the swizzled 32-row block (0-3) of the wave's first B row block
  };
  auto setup = [&](int bid, TileState& ts) {
    const int ci = bid / tpc;
    const int j = bid - ci * tpc;
    ts.chunk = (first_chunk + ci) % num_chunks;
    const int lj = (tpc % 8 == 0) ? (j % 8) * (tpc / 8) + j / 8 : j;
    const int group = lj / (GM * tiles_n);
    const int first_tm = group * GM;
    const int gsz = min(tiles_mc - first_tm, GM);
    const int tm_idx = first_tm + (lj % (GM * tiles_n)) % gsz;
    const int tn_idx = (lj % (GM * tiles_n)) / gsz;
    const int chunk_m0 = ts.chunk * chunk_rows;
    ts.m0 = chunk_m0 + tm_idx * BM;
    ts.m_end = min(ts.m0 + BM, chunk_m0 + chunk_rows);
    ts.n0 = tn_idx * (EPI == EPI_SWIGLU ? HB : BN);
    // lane terms from an opaque copy of the lane index: recomputed per tile rather than kept
    // live through the main loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < T::DA; ++i) {
      // LDS kilobyte wave * DA + i of an A slot holds tile rows 32 wave + 8 i + [0, 8): waves
      // 0-3 fill rows 0-127, waves 4-7 rows 128-255, the rows their own group reads
      const int sidx = (wave * T::DA + i) * 64 + ln;
      const int r = sidx >> 3;
      ts.a_off[i] = (uint32_t)min(ts.m0 + r, M - 1) * (uint32_t)K + (((sidx & 7) ^ swz(r)) * 16);
    }
#pragma unroll
    for (int i = 0; i < T::DB; ++i) {
      const int sidx = (wave * T::DB + i) * 64 + ln;
      const int r = sidx >> 3;
      const uint32_t brow = EPI == EPI_SWIGLU ? (uint32_t)(r < HB ? ts.n0 + r : sg.inter + ts.n0 + (r - HB))
                                              : (uint32_t)min(ts.n0 + r, N - 1);
      ts.b_off[i] = brow * (uint32_t)K + (((sidx & 7) ^ swz(r)) * 16);
    }
    // rows r, r + 32, r + 64, r + 96 of a swizzled 128-row group keep their 4-byte scale groups
    // side by side: one 8-byte load for the wave's two A row blocks, one 16-byte load for the
    // four B row blocks of a 128-column wave or, per lane half, for one of the two groups that
    // the three blocks of a 96-column wave touch (rows past the operand read zero padding or 0;
    // not stored)
    ts.sa_off = scale_base<1>((uint32_t)(ts.m0 + wm * T::WTM + (ln & 31)), nblk4);
    // the wave's first B row (a multiple of 32; fused: its 128 gate or up rows)
    const uint32_t c0 = EPI == EPI_SWIGLU ? (uint32_t)(wn == 0 ? ts.n0 : sg.inter + ts.n0) : (uint32_t)(ts.n0 + wn * T::WTN);
    ts.sbq = (int)(c0 >> 5) & 3;
    if constexpr (SB_TWO_GROUPS)  // past the last group the load reads 0 (resource bound)
      ts.sb_off[0] = scale_base<1>(((c0 >> 7) + (uint32_t)(ln >> 5)) * 128 + (uint32_t)(ln & 31), nblk4);
    else
      ts.sb_off[0] = scale_base<1>(c0 + (uint32_t)(ln & 31), nblk4);
  };
  // loads past the last step go through empty resources: dropped, but counted like the others
  auto issue_a = [&](const TileState& ts, int kt, int slot) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(A, kt < KT ? a_bytes : 0u);
    uint8_t* st = smem + A_RING + slot * T::A_BYTES;
#pragma unroll
    for (int i = 0; i < T::DA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(st + (wave * T::DA + i) * 1024), 16, ts.a_off[i],
                                               (uint32_t)kt * BK, 0, 0);
  };
  auto issue_b = [&](const TileState& ts, int kt, int slot) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(B, kt < KT ? b_bytes : 0u);
    uint8_t* st = smem + B_RING + slot * T::B_BYTES;
#pragma unroll
    for (int i = 0; i < T::DB; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(st + (wave * T::DB + i) * 1024), 16, ts.b_off[i],
                                               (uint32_t)kt * BK, 0, 0);
  };
  // scale registers of one step: the wave's A row blocks, then its B row blocks
  struct Scales {
    u32x2 a;
    uint32_t b[SBW];
  };
  auto load_sa = [&](const TileState& ts, int kt, Scales& sc) {
    const bool live = kt < KT;
    const int so = live ? kt * (int)scale_step<1>() : 0;
    sc.a = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(make_rsrc(As, live ? sa_bytes : 0u), ts.sa_off, so, 0));
  };
  auto load_sb_at = [&](const uint32_t (&sb_off)[NSB], int kt, Scales& sc) {
    const bool live = kt < KT;
    const int so = live ? kt * (int)scale_step<1>() : 0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(Bs, live ? sb_bytes : 0u);
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, sb_off[0], so, 0));
#pragma unroll
    for (int t = 0; t < SBW; ++t) sc.b[t] = v[t];
  };
  auto load_sb = [&](const TileState& ts, int kt, Scales& sc) { load_sb_at(ts.sb_off, kt, sc); };
  // a tile's first loads, in the loop's order (B(s + 1) and the B scales issued last before
  // step s), so that the counts and the compiler's own waits for the scales see the same loads
  // in flight
  auto first_loads = [&](const TileState& ts, Scales& sc) {
    issue_b(ts, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_sa(ts, 0, sc);
    __builtin_amdgcn_sched_barrier(0);
    issue_a(ts, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_b(ts, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    load_sb(ts, 0, sc);
    __builtin_amdgcn_sched_barrier(0);
  };
  // end of a phase: nothing moves across it, and every wave's LDS reads have completed
  auto phase_end = [] {
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  int bid = blockIdx.x;
  if (bid >= total) return;
  // With a multiple of six K steps (and the overlapped epilogue) the ring slots of a tile's
  // first steps are those its predecessor's last steps would fill next: the last two steps
  // then issue the next tile's first loads in place of the dropped ones, and the epilogue
  // issues none (eight waves issuing them at once there kept the address path busy for
  // thousands of cycles).
  // CH: 0, or for chained tiles (K steps even, KT - 1 = CH mod 6) the number of steps after the
  // last whole group of six
  static_assert(CH == 0 || (OVL && (CH == 1 || CH == 3 || CH == 5)), "chained tiles: even K steps, overlapped epilogue");
  constexpr bool CHAIN = CH != 0;
  // chained: the next tile's state is set up a tile ahead (where the matrix pipes idle anyway)
  TileState cur, nxt;
  setup(bid, cur);
  if constexpr (CHAIN) setup(bid + (int)gridDim.x < total ? bid + (int)gridDim.x : bid, nxt);
  Scales sc2[2];
  first_loads(cur, sc2[0]);
  if constexpr (OVL) {
    // 16 stores past the end of an empty resource (dropped): every tile then starts with the
    // same 16 stores behind its first loads. They must stay behind those loads: the compiler
    // may otherwise interleave them, and the first counts would no longer cover the loads.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    const __amdgpu_buffer_rsrc_t none = make_rsrc(C, 0);
#pragma unroll
    for (int i = 0; i < C_STORES; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0x80000000u + 16u * i, 0, 0);
  }

  while (true) {
    const bool has_next = bid + (int)gridDim.x < total;
    const int done_m0 = cur.m0, done_m_end = cur.m_end, done_n0 = cur.n0, done_chunk = cur.chunk;
    // per-lane LDS bases of the fragment reads: A slot 0 (slot 1 at +32 KiB), B slot 0 (slots
    // 1 and 2 at + B_BYTES and + 2 B_BYTES, or slot 2 from a base of its own when it lies beyond
    // the reach of an instruction offset); the block offsets t * 4 KiB and the slot offsets are
    // instruction offsets (below 64 KiB). From an opaque copy of the lane index, per tile.
    int va[2][2], vb[2][2], vb2[2][2];
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      int oa[2][2], ob[2][2];
      frag_offsets<T>(wm, wn, ln & 31, ln >> 5, oa, ob);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          va[kk][h] = A_RING + wm * T::WTM * 128 + oa[kk][h];
          vb[kk][h] = B_RING + wn * T::WTN * 128 + ob[kk][h];
          vb2[kk][h] = vb[kk][h] + 2 * T::B_BYTES;
          if constexpr (FAR_B2)
            asm volatile("" : "+v"(va[kk][h]), "+v"(vb[kk][h]), "+v"(vb2[kk][h]));
          else
            asm volatile("" : "+v"(va[kk][h]), "+v"(vb[kk][h]));
        }
    }
    v16f acc[TN][T::TM];
#pragma unroll
    for (int x = 0; x < TN; ++x)
#pragma unroll
      for (int y = 0; y < T::TM; ++y)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.f;

    // fragments of one 64-K half step (ks) from A slot sa_slot and B slot sb_slot
    auto read_frags = [&](int sa_slot, int sb_slot, int ks, v8i (&af)[T::TM], v8i (&bf)[TN]) {
#pragma unroll
      for (int t = 0; t < T::TM; ++t) {
        const int kk = ks ^ (t & 1);
        const uint8_t* p0 = smem + va[kk][0] + sa_slot * T::A_BYTES + t * 32 * 128;
        const uint8_t* p1 = smem + va[kk][1] + sa_slot * T::A_BYTES + t * 32 * 128;
        const v4i lo = *(const v4i*)p0, hi = *(const v4i*)p1;
        af[t] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int kk = ks ^ (t & 1);
        const int b0 = FAR_B2 && sb_slot == 2 ? vb2[kk][0] : vb[kk][0] + sb_slot * T::B_BYTES;
        const int b1 = FAR_B2 && sb_slot == 2 ? vb2[kk][1] : vb[kk][1] + sb_slot * T::B_BYTES;
        const v4i lo = *(const v4i*)(smem + b0 + t * 32 * 128), hi = *(const v4i*)(smem + b1 + t * 32 * 128);
        bf[t] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };
    // the half step's MFMAs: the instruction takes byte 0 (first 64 K) or 2 (second 64 K) of
    // each scale register, so lanes of block g = 1 shift theirs down by one byte
    auto mma_half = [&](int ks, const v8i (&af)[T::TM], const v8i (&bf)[TN], const Scales& sc) {
      uint32_t as_sel[T::TM], bs_sel[TN];
#pragma unroll
      for (int t = 0; t < T::TM; ++t) as_sel[t] = sc.a[t] >> (8 * g);
      if constexpr (SB_TWO_GROUPS) {
        // every lane gets both groups' dwords of its row (lanes 0-31 loaded the first group,
        // d0-d3, lanes 32-63 the second, e0-e3), then block t's dword is number q + t of
        // d0-d3 e0 e1, chosen by selects on the two bits of q (kept as registers: an indexed
        // form would go through scratch memory)
        const auto s0 = __builtin_amdgcn_permlane32_swap(sc.b[0], sc.b[0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(sc.b[1], sc.b[1], false, false);
        const auto s2 = __builtin_amdgcn_permlane32_swap(sc.b[2], sc.b[2], false, false);
        const auto s3 = __builtin_amdgcn_permlane32_swap(sc.b[3], sc.b[3], false, false);
        uint32_t d0 = s0[0], d1 = s1[0], d2 = s2[0], d3 = s3[0], e0 = s0[1], e1 = s1[1];
        asm volatile("" : "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3), "+v"(e0), "+v"(e1));
        const bool q0 = cur.sbq & 1, q1 = cur.sbq & 2;
        const uint32_t b0 = q1 ? (q0 ? d3 : d2) : (q0 ? d1 : d0);
        const uint32_t b1 = q1 ? (q0 ? e0 : d3) : (q0 ? d2 : d1);
        const uint32_t b2 = q1 ? (q0 ? e1 : e0) : (q0 ? d3 : d2);
        bs_sel[0] = b0 >> (8 * g);
        bs_sel[1] = b1 >> (8 * g);
        bs_sel[2 % TN] = b2 >> (8 * g);
      } else {
#pragma unroll
        for (int t = 0; t < TN; ++t) bs_sel[t] = sc.b[t] >> (8 * g);
      }
#pragma unroll
      for (int x = 0; x < TN; ++x)
#pragma unroll
        for (int y = 0; y < T::TM; ++y) {
          if (ks == 0)
            acc[x][y] = mfma<0>(bf[x], af[y], acc[x][y], (int)bs_sel[x], (int)as_sel[y]);
          else
            acc[x][y] = mfma<2>(bf[x], af[y], acc[x][y], (int)bs_sel[x], (int)as_sel[y]);
        }
    };
    // One 128-K step s (J = s mod 6) as four phases. First memory phase: the fragments, then the
    // A scales of step s + 1 and A(s + 1) (into this group's rows of the slot of step s - 1,
    // which the group has finished reading). Second memory phase: the fragments, then B(s + 2)
    // (into the slot of step s - 1, which both groups have finished reading) and the B scales of
    // step s + 1. In a tile's first step the previous tile's C stores may still be in flight
    // behind B(1) and the B scales of step 0.
    // Mode: 0 any step, 1 the second-to-last step of a chained tile (B(s + 2) is the next tile's
    // B(0)), 2 its last step (every load is the next tile's, and nothing is waited for: this
    // tile's data has landed)
    auto stage = [&](auto Jc, int s, auto First, auto Mode) {
      constexpr int J = decltype(Jc)::value;
      constexpr bool FIRST = decltype(First)::value;
      constexpr int MODE = decltype(Mode)::value;
      constexpr int AS = J & 1, BS = J % 3, CUR = J & 1, NXT = (J + 1) & 1;
      v8i af[T::TM], bf[TN];
      // memory, first half
      read_frags(AS, BS, 0, af, bf);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE == 2) {
        load_sa(nxt, has_next ? 0 : KT, sc2[NXT]);
        __builtin_amdgcn_sched_barrier(0);
        issue_a(nxt, has_next ? 0 : KT, AS ^ 1);
      } else {
        load_sa(cur, s + 1, sc2[NXT]);
        __builtin_amdgcn_sched_barrier(0);
        issue_a(cur, s + 1, AS ^ 1);
      }
      phase_end();
      // compute, first half
      __builtin_amdgcn_s_setprio(1);
      mma_half(0, af, bf, sc2[CUR]);
      __builtin_amdgcn_s_setprio(0);
      phase_end();
      // memory, second half; then B(s + 1) has landed (behind it: the B scales of s, the A
      // scales of s + 1, A(s + 1), B(s + 2) and the B scales of s + 1), before the barrier after
      // which the first group reads it
      read_frags(AS, BS, 1, af, bf);
      __builtin_amdgcn_sched_barrier(0);
      // B(s + 2) goes to slot (J + 2) mod 3; past this tile, the next tile's B(0) and B(1) go to
      // slots 0 and 1, so a chained step fills those with them (slot 2 is left alone)
      constexpr int BT = (J + 2) % 3;
      if constexpr (MODE == 0)
        issue_b(cur, s + 2, BT);
      else if constexpr (BT < 2)
        issue_b(nxt, has_next ? BT : KT, BT);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE == 2)
        load_sb(nxt, has_next ? 0 : KT, sc2[NXT]);
      else
        load_sb(cur, s + 1, sc2[NXT]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE == 2) {
      } else if constexpr (FIRST) {
        wait_vm<C_STORES + 2 * NSB + 1 + T::DA + T::DB>();
      } else {
        wait_vm<2 * NSB + 1 + T::DA + T::DB>();
      }
      phase_end();
      // compute, second half; then A(s + 1) has landed (behind it: B(s + 2) and the B scales of
      // s + 1), before the barrier after which this group reads it
      __builtin_amdgcn_s_setprio(1);
      mma_half(1, af, bf, sc2[CUR]);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MODE != 2) wait_vm<T::DB + NSB>();
      phase_end();
    };

    // B(0), the A scales of step 0 and A(0) have landed; B(1), the B scales of step 0 and the C
    // stores issued after them (the previous tile's, or before the first tile dropped ones) may
    // still be in flight (chained with CH = 3, B(0) was issued last, right before the stores)
    wait_vm<(CH == 3 ? 0 : T::DB + NSB) + C_STORES>();
    phase_end();
    if (grp) phase_end();  // the second group starts one phase late
    // The first step on its own (its count lets the previous tile's C stores stay in flight),
    // then six steps per iteration, left after the last step wherever it falls (a wait count
    // chosen at run time inside a step would split it, and the compiler then spills)
    using No = std::integral_constant<bool, false>;
    using M0 = std::integral_constant<int, 0>;
    stage(std::integral_constant<int, 0>{}, 0, std::integral_constant<bool, true>{}, M0{});
    if constexpr (CHAIN) {
      // whole groups of six, then the last CH steps straight (the last two issuing the next
      // tile's first loads)
      for (int s = 1; s + 6 + CH <= KT; s += 6) {
        stage(std::integral_constant<int, 1>{}, s, No{}, M0{});
        stage(std::integral_constant<int, 2>{}, s + 1, No{}, M0{});
        stage(std::integral_constant<int, 3>{}, s + 2, No{}, M0{});
        stage(std::integral_constant<int, 4>{}, s + 3, No{}, M0{});
        stage(std::integral_constant<int, 5>{}, s + 4, No{}, M0{});
        stage(std::integral_constant<int, 0>{}, s + 5, No{}, M0{});
      }
      // (exits the compiler cannot rule out split the last steps into blocks as in the loop;
      // as one block their fragment registers were spilled)
      int kt_o = KT;
      asm volatile("" : "+s"(kt_o));
      auto tail = [&](auto Jc) {
        constexpr int J = decltype(Jc)::value;
        if constexpr (J <= CH)
          stage(Jc, KT - CH - 1 + J, No{}, std::integral_constant<int, J == CH ? 2 : J == CH - 1 ? 1 : 0>{});
      };
      do {
        tail(std::integral_constant<int, 1>{});
        if (CH == 1 || kt_o < 0) break;
        tail(std::integral_constant<int, 2>{});
        if (kt_o < 0) break;
        tail(std::integral_constant<int, 3>{});
        if (CH == 3 || kt_o < 0) break;
        tail(std::integral_constant<int, 4>{});
        if (kt_o < 0) break;
        tail(std::integral_constant<int, 5>{});
      } while (false);
    } else if (KT > 1) {
      for (int s = 1;; s += 6) {
        stage(std::integral_constant<int, 1>{}, s, No{}, M0{});
        if (s + 1 >= KT) break;
        stage(std::integral_constant<int, 2>{}, s + 1, No{}, M0{});
        if (s + 2 >= KT) break;
        stage(std::integral_constant<int, 3>{}, s + 2, No{}, M0{});
        if (s + 3 >= KT) break;
        stage(std::integral_constant<int, 4>{}, s + 3, No{}, M0{});
        if (s + 4 >= KT) break;
        stage(std::integral_constant<int, 5>{}, s + 4, No{}, M0{});
        if (s + 5 >= KT) break;
        stage(std::integral_constant<int, 0>{}, s + 5, No{}, M0{});
        if (s + 6 >= KT) break;
      }
    }
    if (!grp) phase_end();  // the first group meets the second group's last barrier
    // Every load of this tile has landed (chained, the last ones were waited for a step ago).
    // Nothing may write the epilogue's staging slots (A slot 1, B slot 2) under it: unchained,
    // wait for the dropped loads too; chained, the next tile's loads write A slot 0 and B slots
    // 0 and 1 only, but with one step after the last group (CH = 1) the step before it dropped
    // a B load into slot 2 (11 loads behind it: its B scales, the next tile's A scales, A(0),
    // B(0) and B scales)
    if constexpr (!CHAIN)
      wait_vm<0>();
    else if constexpr (CH == 1)
      wait_vm<3 * NSB + T::DA + T::DB - 1>();
    // the scale registers stay live past the loop: otherwise the compiler sinks each step's scale
    // loads into the next step (their only use, behind an early exit), right before the MFMAs.
    // Chained, set 0 holds the next tile's first scales, still in flight: a use here would wait
    // for them and for every first load issued before them
    if constexpr (!CHAIN) {
      asm volatile("" ::"v"(sc2[0].a));
#pragma unroll
      for (int t = 0; t < SBW; ++t) asm volatile("" ::"v"(sc2[0].b[t]));
    }
    asm volatile("" ::"v"(sc2[1].a));
#pragma unroll
    for (int t = 0; t < SBW; ++t) asm volatile("" ::"v"(sc2[1].b[t]));

    block_barrier();  // every wave's loads have landed and its reads are done
    int tid_e = tid;
    asm volatile("" : "+v"(tid_e));
    const int e32 = tid_e & 31, eg = (tid_e >> 5) & 1;
    const int nbid = bid + (int)gridDim.x;
    if constexpr (EPI == EPI_SWIGLU) {
      // every load has landed (unchained); the fused epilogue stages through the whole LDS
      swiglu_epilogue<T>(smem, acc, wm, wn, e32, eg, tid_e, done_m0, done_m_end, done_n0, sg);
      if (has_next) {
        block_barrier();  // every wave has read its part of the staged band
        setup(nbid, cur);
        first_loads(cur, sc2[0]);
      }
    } else if constexpr (OVL) {
      // ---- epilogue, with the next tile's first loads issued half-way.
      // Quarter qd = (y, h): tile rows 64 wm + 32 y + [0, 32) of every wm and tile columns
      // 128 wn + 64 h + [0, 64) of both wn, staged as 128 rows of 256 bytes (row 32 wm + l32,
      // 16-byte chunk 8 wn + column / 8 within the half) with the chunk index xor-ed with
      // row & 7, so that the 8-byte writes (32 rows) and the 16-byte reads (4 whole rows) of one
      // instruction both spread evenly over the banks.
      auto stage_quarter = [&](int qd, uint8_t* st) {
        const int y = qd >> 1, h = qd & 1;
        const int rq = wm * 32 + e32;
#pragma unroll
        for (int xx = 0; xx < 2; ++xx) {
          const int x = 2 * h + xx;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int chunk = wn * 8 + xx * 4 + q;
            const uint32_t lo = pack_bf16x2(acc[x][y][4 * q + 0], acc[x][y][4 * q + 1]);
            const uint32_t hi = pack_bf16x2(acc[x][y][4 * q + 2], acc[x][y][4 * q + 3]);
            // the next tile's loads in flight write A slot 0 and B slots 0 and 1 only
            lds_store_b64_unordered(st + rq * 256 + ((chunk ^ (rq & 7)) * 16) + eg * 8, u32x2{lo, hi});
          }
        }
      };
      // the first two quarters (half of the accumulators) go to LDS before the next tile's
      // loads are issued, so that its offsets and this tile's remaining accumulators fit
      stage_quarter(0, stage0);
      stage_quarter(1, stage1);
      if constexpr (CHAIN) {
        // the next tile's loads are in flight but for B(0) (CH = 3) or B(1) (CH = 1), whose slot
        // the last step was reading; set up the tile after it
        cur = nxt;
        if constexpr (CH == 3) issue_b(cur, has_next ? 0 : KT, 0);
        if constexpr (CH == 1) issue_b(cur, has_next ? 1 : KT, 1);
        const int nnbid = nbid + (int)gridDim.x;
        setup(nnbid < total ? nnbid : nbid, nxt);
      } else if (has_next) {
        setup(nbid, cur);
        first_loads(cur, sc2[0]);
      }
      // C through a resource over this tile's rows: elements past the last row or column get
      // an offset past its end and are dropped, so every wave issues the same 16 stores
      const uint32_t c_bytes = (uint32_t)(done_m_end - done_m0) * (uint32_t)ldc * 2u;
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(C + (int64_t)done_m0 * ldc, c_bytes);
      auto store_quarter = [&](int qd, const uint8_t* st) {
        const int y = qd >> 1, h = qd & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = tid_e + i * T::NT;
          const int rq = p >> 4, chunk = p & 15;
          const u32x4 v = *(const u32x4*)(st + rq * 256 + ((chunk ^ (rq & 7)) * 16));
          const int r = (rq >> 5) * 64 + y * 32 + (rq & 31);  // tile row
          const int n = done_n0 + (chunk >> 3) * 128 + h * 64 + (chunk & 7) * 8;
          const bool ok = done_m0 + r < done_m_end && n < N;
          const uint32_t off = ok ? ((uint32_t)r * (uint32_t)ldc + (uint32_t)n) * 2u : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 2);
        }
      };
      block_barrier();
      store_quarter(0, stage0);
      store_quarter(1, stage1);
      block_barrier();
      stage_quarter(2, stage0);
      stage_quarter(3, stage1);
      block_barrier();
      store_quarter(2, stage0);
      store_quarter(3, stage1);
    } else {
      // ---- epilogue: the BF16 tile staged in LDS (rows padded by 16 bytes, 8-byte halves
      // swapped on alternate row groups), then full-line 16-byte stores; the next tile's first
      // loads once every wave has read its part
#pragma unroll
      for (int x = 0; x < TN; ++x) {
#pragma unroll
        for (int y = 0; y < T::TM; ++y) {
          const int r = wm * T::WTM + y * 32 + e32;
          const int gs = eg ^ (((r >> 3) ^ (r >> 4)) & 1);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = wn * T::WTN + x * 32 + 8 * q + 4 * gs;
            const uint32_t lo = pack_bf16x2(acc[x][y][4 * q + 0], acc[x][y][4 * q + 1]);
            const uint32_t hi = pack_bf16x2(acc[x][y][4 * q + 2], acc[x][y][4 * q + 3]);
            *(uint2*)(smem + r * T::C_STRIDE + c * 2) = make_uint2(lo, hi);
          }
        }
      }
      block_barrier();
      constexpr int SEGS = BN / 8;  // 16-byte segments per row
#pragma unroll 4
      for (int p = tid_e; p < BM * SEGS; p += T::NT) {
        const int r = p / SEGS;
        const int c8 = (p % SEGS) * 8;
        const int m = done_m0 + r;
        const int n = done_n0 + c8;
        if (m >= done_m_end || n >= N) continue;
        uint4 v = *(const uint4*)(smem + r * T::C_STRIDE + c8 * 2);
        if (((r >> 3) ^ (r >> 4)) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
        __builtin_nontemporal_store(*(const u32x4*)&v, (u32x4*)(C + (int64_t)m * ldc + n));
      }
      if (has_next) {
        block_barrier();  // every wave has read its part of the staged tile
        setup(nbid, cur);
        first_loads(cur, sc2[0]);
      }
    }

    if (chunk_done != nullptr) {
      __threadfence();  // this thread's C stores are visible device-wide
      __syncthreads();
      if (tid == 0) atomicAdd(chunk_done + done_chunk, 1);
    }
    if (!has_next) break;
    bid = nbid;
  }
  // (chained, the last tile's last steps issued dropped loads that write no LDS this workgroup
  // reads; they complete before its waves end)
  wait_vm<0>();
#endif
}

// Tile configurations: output tile, wave grid, LDS stages.
using TileL = Tile<256, 256, 4, 2, 2>;  // 8 waves of 64 x 128; large problems
using TileLR = Tile<256, 256, 4, 2, 2, true>;  // the same with the split ring (swizzled scales)
using TileN = Tile<256, 192, 4, 2, 2>;  // 8 waves of 64 x 96; when 256 x 256 leaves a round part-empty
using TileNR = Tile<256, 192, 4, 2, 2, true>;  // the same as two wave groups (swizzled scales)
using TileW = Tile<128, 192, 4, 2, 3>;  // 8 waves of 32 x 96
using TileQ = Tile<192, 192, 3, 2, 3>;  // 6 waves of 64 x 96
using TileR = Tile<96, 192, 3, 2, 4>;   // 6 waves of 32 x 96
using TileM = Tile<128, 128, 4, 2, 4>;  // 8 waves of 32 x 64
using TileS = Tile<64, 128, 2, 4, 4>;   // 8 waves of 32 x 32
using TileT = Tile<32, 128, 1, 4, 4>;   // 4 waves of 32 x 32; a few rows per chunk
using TileD = Tile<32, 32, 1, 1, 8, false, true>;  // one wave, fragments loaded to registers

constexpr int REF_CUS = 256;  // compute units the tile choice is made for (MI355X)

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return REF_CUS;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = REF_CUS;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int64_t tile_count(int64_t m, int64_t n, int num_chunks, int bm, int bn) {
  return (int64_t)num_chunks * ((m / num_chunks + bm - 1) / bm) * ((n + bn - 1) / bn);
}

enum { CFG_L, CFG_N, CFG_Q, CFG_W, CFG_R, CFG_M, CFG_S, CFG_T, CFG_D };

// Tile choice by estimated makespan: rounds of workgroups over the compute units times the
// time of one tile's 128-K step, measured per configuration on MI355X (N = 6144 sweeps, in
// microseconds; smaller tiles take less time per step but need more rounds). Among equal
// estimates the configuration with more tiles wins (more workgroups in flight). A tile must
// fit in a chunk's rows (the 32-row tile takes any chunk).
struct CfgInfo {
  int id, bm, bn;
  double step_us;
};
constexpr CfgInfo kCfgs[] = {{CFG_L, 256, 256, 2.0},  {CFG_N, 256, 192, 2.0},  {CFG_Q, 192, 192, 1.67},
                             {CFG_W, 128, 192, 1.23}, {CFG_R, 96, 192, 1.10},  {CFG_M, 128, 128, 0.96},
                             {CFG_S, 64, 128, 0.73},  {CFG_T, 32, 128, 0.40}};

int pick_config(int64_t m, int64_t n, int num_chunks) {
  const int64_t rows = m / num_chunks;
  int best = CFG_T;
  double best_span = 0.0;
  int64_t best_tiles = 0;
  for (const CfgInfo& c : kCfgs) {
    if (c.id != CFG_T && rows < c.bm) continue;  // the 32-row tile takes any chunk
    const int64_t tiles = tile_count(m, n, num_chunks, c.bm, c.bn);
    const double span = (double)((tiles + REF_CUS - 1) / REF_CUS) * c.step_us;
    if (best_tiles == 0 || span < best_span * 0.999 || (span <= best_span * 1.001 && tiles > best_tiles)) {
      best = c.id;
      best_span = span;
      best_tiles = tiles;
    }
  }
  return best;
}

// The BF16-output GEMM of at most 32 rows in one chunk (decode sizes) takes one-wave 32 x 32
// tiles that load their fragments straight into registers: four times the workgroups of the
// 32 x 128 tile (whose N / 128 workgroups leave most CUs idle), each without LDS stages or
// barriers (M = 1, 8 and 32 at K = 2048: 9.9, 10.6 and 12.7 us against 12.6, 13.0 and
// 14.6). Once the 32 x 128 tile has more workgroups it is faster: its LDS-DMA loads cover
// 8 rows x 128 bytes per instruction where a register load covers 32 rows x 32 bytes, and
// the extra requests cost more than the barriers saved (M = 64: 16.8 against 14.1 us; M = 128
// in four chunks of 32 rows: 20.9 against 12.1 us).
//
// With both scales swizzled (and chunks on 64-row boundaries) the 256 x 256 and 256 x 192 tiles
// run the two-group kernel, whose K step costs less than the staged tiles' model assumes; where
// the model picks the staged 192 x 192 tile and a chunk has at least 256 rows, the two-group
// 256 x 192 tile is faster (M = 1536: 28.6 / 38.3 against 29.4 / 40.0 us at K = 2048 / 3072;
// M = 3072: 48.9 / 68.5 against 54.4 / 76.4 us; 4 chunks, N = 6144). The choice depends on the
// layouts only, not on the buffers' alignment, so that the tile count per chunk is known to the
// caller beforehand (mxfp8_gemm_tiles_per_chunk).
bool two_group_layouts(int a_layout, int b_layout, int64_t m, int num_chunks) {
  return a_layout == 1 && b_layout == 1 && (num_chunks == 1 || (m / num_chunks) % 64 == 0);
}

int pick_config_bf16(int64_t m, int64_t n, int num_chunks, bool two_group) {
  int c = pick_config(m, n, num_chunks);
  if (two_group && c == CFG_Q && m / num_chunks >= 256) c = CFG_N;
  return c == CFG_T && num_chunks == 1 && m <= 32 ? CFG_D : c;
}

template <class T, int EPI = EPI_BF16>
hipError_t launch_cfg(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b, const uint8_t* bs,
                      int b_layout, int64_t m, int64_t n, int64_t k, uint16_t* c, int64_t ldc, int num_chunks,
                      int first_chunk, int* chunk_done, hipStream_t stream, SwiGluOut sg = SwiGluOut{}) {
  const int64_t tiles = tile_count(m, n, num_chunks, T::BM, T::BN);
  // one-wave direct tiles: up to eight workgroups per compute unit; the others: one
  const int64_t cap = (T::DIRECT ? 8 : 1) * (int64_t)device_cu_count();
  const int64_t grid = tiles < cap ? tiles : cap;
  const int wide = ((uintptr_t)c % 16 == 0 && ldc % 8 == 0) ? 1 : 0;
  const dim3 g((unsigned)grid), blk(T::NT);
  const int M = (int)m, N = (int)n, K = (int)k, L = (int)ldc;
  if (a_layout == 0 && b_layout == 0)
    gemm_kernel<T, 0, 0, EPI><<<g, blk, 0, stream>>>(a, as, b, bs, c, M, N, K, L, num_chunks, first_chunk, chunk_done, wide, sg);
  else if (a_layout == 0 && b_layout == 1)
    gemm_kernel<T, 0, 1, EPI><<<g, blk, 0, stream>>>(a, as, b, bs, c, M, N, K, L, num_chunks, first_chunk, chunk_done, wide, sg);
  else if (a_layout == 1 && b_layout == 0)
    gemm_kernel<T, 1, 0, EPI><<<g, blk, 0, stream>>>(a, as, b, bs, c, M, N, K, L, num_chunks, first_chunk, chunk_done, wide, sg);
  else
    gemm_kernel<T, 1, 1, EPI><<<g, blk, 0, stream>>>(a, as, b, bs, c, M, N, K, L, num_chunks, first_chunk, chunk_done, wide, sg);
  return hipGetLastError();
}

// The split ring reads the swizzled scales of a wave's rows with single wide loads: both
// operands' scales swizzled and 16-byte aligned, chunks starting on 64-row boundaries.
bool split_ring_fits(const uint8_t* as, int a_layout, const uint8_t* bs, int b_layout, int64_t m, int num_chunks) {
  return a_layout == 1 && b_layout == 1 && (uintptr_t)as % 16 == 0 && (uintptr_t)bs % 16 == 0 &&
         (num_chunks == 1 || (m / num_chunks) % 64 == 0);
}

// The two-group BF16 kernel (swizzled, 16-byte aligned scales on 64-row chunk boundaries, checked
// by the caller): output in whole 16-byte segments, at least two K steps, tile offsets in 32
// bits. Returns false (launching nothing) when the output does not qualify.
template <class T, int EPI = EPI_BF16>
bool launch_two_group(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs, int64_t m, int64_t n,
                      int64_t k, uint16_t* c, int64_t ldc, int num_chunks, int first_chunk, int* chunk_done,
                      hipStream_t stream, hipError_t& err, SwiGluOut sg = SwiGluOut{}) {
  if constexpr (EPI == EPI_SWIGLU) {
    // fused dense GEMM1: tiles of BN / 2 gate and BN / 2 up columns, no chunk counters
    if (!(k >= 2 * BK && sg.inter % (T::BN / 2) == 0 && n == 2 * (int64_t)sg.inter)) return false;
    const int64_t tiles = tile_count(m, sg.inter * 2, num_chunks, T::BM, T::BN);
    const int64_t grid = tiles < device_cu_count() ? tiles : device_cu_count();
    gemm_pingpong_bf16_kernel<T, 0, EPI_SWIGLU><<<dim3((unsigned)grid), dim3(T::NT), 0, stream>>>(
        a, as, b, bs, nullptr, (int)m, (int)n, (int)k, 0, num_chunks, first_chunk, nullptr, sg);
    err = hipGetLastError();
    return true;
  } else {
    const bool wide = (uintptr_t)c % 16 == 0 && ldc % 8 == 0;
    if (!(k >= 2 * BK && n % 8 == 0 && wide && (int64_t)ldc * 2 * T::BM < (1ll << 31))) return false;
    const int64_t tiles = tile_count(m, n, num_chunks, T::BM, T::BN);
    const int64_t grid = tiles < device_cu_count() ? tiles : device_cu_count();
    // with the overlapped epilogue and an even number of K steps, consecutive tiles chain their
    // loads; the variant follows the number of steps after the last whole group of six
    const int kt = (int)(k / BK);
    constexpr int CH5 = T::BN == 256 ? 5 : 0, CH3 = T::BN == 256 ? 3 : 0, CH1 = T::BN == 256 ? 1 : 0;
    if (T::BN == 256 && kt % 6 == 0)
      gemm_pingpong_bf16_kernel<T, CH5><<<dim3((unsigned)grid), dim3(T::NT), 0, stream>>>(
          a, as, b, bs, c, (int)m, (int)n, (int)k, (int)ldc, num_chunks, first_chunk, chunk_done);
    else if (T::BN == 256 && kt % 6 == 4)
      gemm_pingpong_bf16_kernel<T, CH3><<<dim3((unsigned)grid), dim3(T::NT), 0, stream>>>(
          a, as, b, bs, c, (int)m, (int)n, (int)k, (int)ldc, num_chunks, first_chunk, chunk_done);
    else if (T::BN == 256 && kt % 6 == 2)
      gemm_pingpong_bf16_kernel<T, CH1><<<dim3((unsigned)grid), dim3(T::NT), 0, stream>>>(
          a, as, b, bs, c, (int)m, (int)n, (int)k, (int)ldc, num_chunks, first_chunk, chunk_done);
    else
      gemm_pingpong_bf16_kernel<T, 0><<<dim3((unsigned)grid), dim3(T::NT), 0, stream>>>(
          a, as, b, bs, c, (int)m, (int)n, (int)k, (int)ldc, num_chunks, first_chunk, chunk_done);
    err = hipGetLastError();
    return true;
  }
}

template <int EPI>
hipError_t launch_split(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs, int64_t m, int64_t n,
                        int64_t k, uint16_t* c, int64_t ldc, int num_chunks, int first_chunk, int* chunk_done,
                        hipStream_t stream, SwiGluOut sg = SwiGluOut{}) {
  using T = TileLR;
  const int64_t tiles = tile_count(m, n, num_chunks, T::BM, T::BN);
  const int64_t grid = tiles < device_cu_count() ? tiles : device_cu_count();
  const int wide = ((uintptr_t)c % 16 == 0 && ldc % 8 == 0) ? 1 : 0;
  hipError_t err = hipSuccess;
  if (EPI == EPI_BF16 &&
      launch_two_group<T>(a, as, b, bs, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream, err))
    return err;
  if (EPI == EPI_SWIGLU && num_chunks == 1 &&
      launch_two_group<T, EPI_SWIGLU>(a, as, b, bs, m, n, k, nullptr, 0, 1, 0, nullptr, stream, err, sg))
    return err;
  gemm_kernel<T, 1, 1, EPI><<<dim3((unsigned)grid), dim3(T::NT), 0, stream>>>(
      a, as, b, bs, c, (int)m, (int)n, (int)k, (int)ldc, num_chunks, first_chunk, chunk_done, wide, sg);
  return hipGetLastError();
}

}  // namespace

GemmShape gemm_pick_shape(int64_t m, int64_t n, int num_chunks, int a_layout, int b_layout) {
  switch (pick_config_bf16(m, n, num_chunks, two_group_layouts(a_layout, b_layout, m, num_chunks))) {
    case CFG_L: return GemmShape{TileL::BM, TileL::BN};
    case CFG_N: return GemmShape{TileN::BM, TileN::BN};
    case CFG_Q: return GemmShape{TileQ::BM, TileQ::BN};
    case CFG_R: return GemmShape{TileR::BM, TileR::BN};
    case CFG_W: return GemmShape{TileW::BM, TileW::BN};
    case CFG_M: return GemmShape{TileM::BM, TileM::BN};
    case CFG_S: return GemmShape{TileS::BM, TileS::BN};
    case CFG_D: return GemmShape{TileD::BM, TileD::BN};
    default: return GemmShape{TileT::BM, TileT::BN};
  }
}

hipError_t launch_gemm_silu_mul_quant(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* w,
                                      const uint8_t* ws, int w_layout, int64_t m, int64_t inter, int64_t k,
                                      uint8_t* q, uint8_t* s_lin, uint8_t* s_swz, hipStream_t stream) {
  const SwiGluOut sg{q, s_lin, s_swz, (int)inter};
  const int64_t n = 2 * inter;  // B rows; tile counts match whenever inter is a multiple of BN/2
  hipError_t e;
  int cfg = pick_config(m, n, 1);
  if (two_group_layouts(a_layout, w_layout, m, 1) && cfg == CFG_Q && m >= 256) cfg = CFG_N;  // as for BF16
  switch (cfg) {
    case CFG_L:
      if (split_ring_fits(as, a_layout, ws, w_layout, m, 1) && inter % 128 == 0)
        e = launch_split<EPI_SWIGLU>(a, as, w, ws, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg);
      else
        e = launch_cfg<TileL, EPI_SWIGLU>(a, as, a_layout, w, ws, w_layout, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg);
      break;
    case CFG_N:
      if (!(split_ring_fits(as, a_layout, ws, w_layout, m, 1) &&
            launch_two_group<TileNR, EPI_SWIGLU>(a, as, w, ws, m, n, k, nullptr, 0, 1, 0, nullptr, stream, e, sg)))
        e = launch_cfg<TileN, EPI_SWIGLU>(a, as, a_layout, w, ws, w_layout, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg);
      break;
    case CFG_Q: e = launch_cfg<TileQ, EPI_SWIGLU>(a, as, a_layout, w, ws, w_layout, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg); break;
    case CFG_R: e = launch_cfg<TileR, EPI_SWIGLU>(a, as, a_layout, w, ws, w_layout, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg); break;
    case CFG_W: e = launch_cfg<TileW, EPI_SWIGLU>(a, as, a_layout, w, ws, w_layout, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg); break;
    case CFG_M: e = launch_cfg<TileM, EPI_SWIGLU>(a, as, a_layout, w, ws, w_layout, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg); break;
    case CFG_S: e = launch_cfg<TileS, EPI_SWIGLU>(a, as, a_layout, w, ws, w_layout, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg); break;
    default: e = launch_cfg<TileT, EPI_SWIGLU>(a, as, a_layout, w, ws, w_layout, m, n, k, nullptr, 0, 1, 0, nullptr, stream, sg); break;
  }
  if (e != hipSuccess) return e;
  if (s_swz) e = launch_swizzle_pad_zero(s_swz, m, inter, stream);
  return e;
}

hipError_t launch_gemm(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b,
                       const uint8_t* bs, int b_layout, int64_t m, int64_t n, int64_t k, uint16_t* c,
                       int64_t ldc, int num_chunks, int first_chunk, int* chunk_done, hipStream_t stream) {
  switch (pick_config_bf16(m, n, num_chunks, two_group_layouts(a_layout, b_layout, m, num_chunks))) {
    case CFG_L:
      if (split_ring_fits(as, a_layout, bs, b_layout, m, num_chunks))
        return launch_split<EPI_BF16>(a, as, b, bs, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
      return launch_cfg<TileL>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
    case CFG_N: {
      hipError_t err = hipSuccess;
      if (split_ring_fits(as, a_layout, bs, b_layout, m, num_chunks) &&
          launch_two_group<TileNR>(a, as, b, bs, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream, err))
        return err;
      return launch_cfg<TileN>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
    }
    case CFG_Q:
      return launch_cfg<TileQ>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
    case CFG_R:
      return launch_cfg<TileR>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
    case CFG_W:
      return launch_cfg<TileW>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
    case CFG_M:
      return launch_cfg<TileM>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
    case CFG_S:
      return launch_cfg<TileS>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
    case CFG_D:
      return launch_cfg<TileD>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
    default:
      return launch_cfg<TileT>(a, as, a_layout, b, bs, b_layout, m, n, k, c, ldc, num_chunks, first_chunk, chunk_done, stream);
  }
}

}  // namespace mxfp8
