// gemm.hip - MXFP8 block-scaled GEMM with BF16 output on gfx950 scaled MFMA.
//
//   C[m,n] = BF16( sum_kb 2^(sa[m,kb]-127) 2^(sb[n,kb]-127) sum_{i<32} A[m,32kb+i] B[n,32kb+i] )
//
// The per-rank GEMM of the o_proj / down_proj GEMM-RS path (vLLM PR #64659, "GEMM-RS
// microbenchmark", N = 6144, K = 2048 / 3072), with the output written in M-row chunks that
// match one rank's reduce-scatter shard ("Overview", "Details").
//
// Design (CDNA4):
//  * One workgroup = 4 waves (2 x 2) computes a BM x BN output tile; each wave owns a
//    (BM/2) x (BN/2) sub-tile made of 32x32 MFMA blocks accumulated in fp32.
//  * V_MFMA_SCALE_F32_32X32X64_F8F6F4 applies the UE8M0 block scales inside the instruction.
//    Operand layout of that instruction (32 rows x 64 K per operand): lane l holds row l%32;
//    with g = l/32, its bytes 0..15 are K 16g..16g+15 and bytes 16..31 are K 32+16g..32+16g+15.
//    The scale of (row r, 32-block b) comes from lane r + 32b, byte selected by OPSEL.
//    Result lane l, register v: column l%32, row 8(v/4) + 4(l/32) + v%4.
//  * The B tile (output columns n) is fed as the instruction's first operand and the A tile as
//    the second, so each lane ends up with runs of 4 consecutive n of one output row m and the
//    epilogue stores 8 bytes per run.
//  * K advances 128 bytes per stage. Stages are double-buffered in LDS and filled directly from
//    global memory with 16-byte LDS-DMA loads (global_load_lds_dwordx4). A row of a stage is
//    8 chunks of 16 bytes; chunk c of row r sits in slot c ^ ((r ^ (r >> 3)) & 7), so the 16
//    consecutive rows one ds_read_b128 touches spread over all banks.
//  * The 4 scale bytes of a row for one stage form one aligned dword in both scale layouts;
//    each lane loads the dwords of its rows one stage ahead and keeps the two bytes it needs.
//  * Tile order: chunk by chunk from first_chunk; inside a chunk every XCD (workgroups are
//    dispatched round-robin over 8 XCDs) gets a contiguous run of tiles, grouped GM tile-rows
//    tall so that concurrently running tiles share A and B panels in that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace mxfp8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 128;  // K bytes per stage
constexpr int NT = 256;  // 4 waves
constexpr int GM = 4;    // tile-rows per group

template <int BM, int BN>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;    // wave sub-tile
  static constexpr int TM = WM / 32, TN = WN / 32;  // MFMA blocks per wave
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Byte offset, inside one stage's A or B region, of logical 16-byte chunk c of row r.
__device__ __forceinline__ int lds_off(int r, int c) { return (r * 8 + (c ^ swz(r))) * 16; }

// Scaled MFMA with compile-time byte selectors.
template <int SEL>
__device__ __forceinline__ v16f mfma(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, sa, SEL, sb);
}

// Offset of the 4-byte scale group (row r, stage kt) in the given layout; nblk4 = K/128.
template <int LAYOUT>
__device__ __forceinline__ uint32_t scale_dword_off(uint32_t r, uint32_t kt, uint32_t nblk4) {
  if (LAYOUT == 0) return (r * nblk4 + kt) * 4;
  return ((r >> 7) * nblk4 + kt) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4;
}

// Issue the LDS-DMA loads of one R-row x 128-byte operand tile: R/8 instructions of 1 KiB,
// R/32 per wave. src_off[i] is the lane's byte offset (row * K + chunk * 16) for instruction i.
template <int R>
__device__ __forceinline__ void issue_tile(const uint8_t* __restrict__ base, const uint32_t* src_off,
                                           uint32_t k0, uint8_t* lds_region, int wave) {
#pragma unroll
  for (int i = 0; i < R / 32; ++i) {
    const int inst = wave * (R / 32) + i;
    __builtin_amdgcn_global_load_lds((const void*)(base + src_off[i] + k0),
                                     (lds_void*)(lds_region + inst * 1024), 16, 0, 0);
  }
}

template <int BM, int BN, int A_LAYOUT, int B_LAYOUT>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(const uint8_t* __restrict__ A,
                                                     const uint8_t* __restrict__ As,
                                                     const uint8_t* __restrict__ B,
                                                     const uint8_t* __restrict__ Bs,
                                                     uint16_t* __restrict__ C, int M, int N, int K,
                                                     int ldc, int num_chunks, int first_chunk,
                                                     int* __restrict__ chunk_done) {
  using T = Tile<BM, BN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;

  // ---- tile coordinates: chunk-major, XCD-contiguous, grouped
  const int chunk_rows = M / num_chunks;
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_mc = (chunk_rows + BM - 1) / BM;
  const int tpc = tiles_mc * tiles_n;
  const int bid = blockIdx.x;
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
  const int n0 = tn_idx * BN;

  // ---- per-lane LDS-DMA source offsets (rows clamped into the operand; surplus rows unused)
  uint32_t a_off[BM / 32], b_off[BN / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int s = (wave * (BM / 32) + i) * 64 + lane;
    const int r = s >> 3;
    const int c = (s & 7) ^ swz(r);
    a_off[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + c * 16;
  }
#pragma unroll
  for (int i = 0; i < BN / 32; ++i) {
    const int s = (wave * (BN / 32) + i) * 64 + lane;
    const int r = s >> 3;
    const int c = (s & 7) ^ swz(r);
    b_off[i] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K + c * 16;
  }

  // ---- per-lane scale rows
  const uint32_t nblk4 = (uint32_t)K / 128;
  uint32_t a_srow[T::TM], b_srow[T::TN];
#pragma unroll
  for (int t = 0; t < T::TM; ++t) a_srow[t] = (uint32_t)min(m0 + wm * T::WM + t * 32 + l32, M - 1);
#pragma unroll
  for (int t = 0; t < T::TN; ++t) b_srow[t] = (uint32_t)min(n0 + wn * T::WN + t * 32 + l32, N - 1);

  v16f acc[T::TN][T::TM];
#pragma unroll
  for (int x = 0; x < T::TN; ++x)
#pragma unroll
    for (int y = 0; y < T::TM; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][y][v] = 0.f;

  const int KT = K / BK;
  uint32_t asc[T::TM], bsc[T::TN];

  // prologue: stage 0
  issue_tile<BM>(A, a_off, 0, smem, wave);
  issue_tile<BN>(B, b_off, 0, smem + T::A_BYTES, wave);
#pragma unroll
  for (int t = 0; t < T::TM; ++t) asc[t] = *(const uint32_t*)(As + scale_dword_off<A_LAYOUT>(a_srow[t], 0, nblk4));
#pragma unroll
  for (int t = 0; t < T::TN; ++t) bsc[t] = *(const uint32_t*)(Bs + scale_dword_off<B_LAYOUT>(b_srow[t], 0, nblk4));

  for (int kt = 0; kt < KT; ++kt) {
    uint8_t* cur = smem + (kt & 1) * T::STAGE;
    uint8_t* nxt = smem + ((kt + 1) & 1) * T::STAGE;
    // this stage's loads have landed in LDS for every wave; the other buffer is free
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // this lane's scale bytes for the stage: byte 0 -> block g (first MFMA), byte 2 -> block 2+g
    uint32_t as_sel[T::TM], bs_sel[T::TN];
#pragma unroll
    for (int t = 0; t < T::TM; ++t) as_sel[t] = (asc[t] >> (8 * g)) & 0x00FF00FFu;
#pragma unroll
    for (int t = 0; t < T::TN; ++t) bs_sel[t] = (bsc[t] >> (8 * g)) & 0x00FF00FFu;

    if (kt + 1 < KT) {
      const uint32_t k0 = (uint32_t)(kt + 1) * BK;
      issue_tile<BM>(A, a_off, k0, nxt, wave);
      issue_tile<BN>(B, b_off, k0, nxt + T::A_BYTES, wave);
#pragma unroll
      for (int t = 0; t < T::TM; ++t)
        asc[t] = *(const uint32_t*)(As + scale_dword_off<A_LAYOUT>(a_srow[t], kt + 1, nblk4));
#pragma unroll
      for (int t = 0; t < T::TN; ++t)
        bsc[t] = *(const uint32_t*)(Bs + scale_dword_off<B_LAYOUT>(b_srow[t], kt + 1, nblk4));
    }

    const uint8_t* a_lds = cur;
    const uint8_t* b_lds = cur + T::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i af[T::TM], bf[T::TN];
#pragma unroll
      for (int t = 0; t < T::TM; ++t) {
        const int r = wm * T::WM + t * 32 + l32;
        const v4i lo = *(const v4i*)(a_lds + lds_off(r, 4 * ks + g));
        const v4i hi = *(const v4i*)(a_lds + lds_off(r, 4 * ks + 2 + g));
        af[t] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int t = 0; t < T::TN; ++t) {
        const int r = wn * T::WN + t * 32 + l32;
        const v4i lo = *(const v4i*)(b_lds + lds_off(r, 4 * ks + g));
        const v4i hi = *(const v4i*)(b_lds + lds_off(r, 4 * ks + 2 + g));
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
    }
  }

  // ---- epilogue: lane holds C[m = row0 + l32][n = col0 + 8*(v/4) + 4*g + v%4]
#pragma unroll
  for (int x = 0; x < T::TN; ++x) {
#pragma unroll
    for (int y = 0; y < T::TM; ++y) {
      const int m = m0 + wm * T::WM + y * 32 + l32;
      if (m >= m_end) continue;
      uint16_t* crow = C + (int64_t)m * ldc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * T::WN + x * 32 + 8 * q + 4 * g;
        const uint32_t b0 = f32_to_bf16_rne(acc[x][y][4 * q + 0]);
        const uint32_t b1 = f32_to_bf16_rne(acc[x][y][4 * q + 1]);
        const uint32_t b2 = f32_to_bf16_rne(acc[x][y][4 * q + 2]);
        const uint32_t b3 = f32_to_bf16_rne(acc[x][y][4 * q + 3]);
        if (n + 3 < N) {
          *(uint2*)(crow + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
          if (n + 0 < N) crow[n + 0] = (uint16_t)b0;
          if (n + 1 < N) crow[n + 1] = (uint16_t)b1;
          if (n + 2 < N) crow[n + 2] = (uint16_t)b2;
        }
      }
    }
  }

  if (chunk_done != nullptr) {
    __threadfence();  // this thread's C stores are visible device-wide
    __syncthreads();
    if (tid == 0) atomicAdd(chunk_done + chunk, 1);
  }
}

template <int BM, int BN>
hipError_t launch_shape(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b, const uint8_t* bs,
                        int b_layout, int m, int n, int k, uint16_t* c, int ldc, int num_chunks, int first_chunk,
                        int* chunk_done, hipStream_t stream) {
  const int chunk_rows = m / num_chunks;
  const int64_t tiles = (int64_t)num_chunks * ((chunk_rows + BM - 1) / BM) * ((n + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(NT);
  if (a_layout == 0 && b_layout == 0)
    gemm_kernel<BM, BN, 0, 0><<<grid, block, 0, stream>>>(a, as, b, bs, c, m, n, k, ldc, num_chunks, first_chunk, chunk_done);
  else if (a_layout == 0 && b_layout == 1)
    gemm_kernel<BM, BN, 0, 1><<<grid, block, 0, stream>>>(a, as, b, bs, c, m, n, k, ldc, num_chunks, first_chunk, chunk_done);
  else if (a_layout == 1 && b_layout == 0)
    gemm_kernel<BM, BN, 1, 0><<<grid, block, 0, stream>>>(a, as, b, bs, c, m, n, k, ldc, num_chunks, first_chunk, chunk_done);
  else
    gemm_kernel<BM, BN, 1, 1><<<grid, block, 0, stream>>>(a, as, b, bs, c, m, n, k, ldc, num_chunks, first_chunk, chunk_done);
  return hipGetLastError();
}

}  // namespace

GemmShape gemm_pick_shape(int64_t m, int64_t n, int num_chunks) {
  (void)m;
  (void)n;
  (void)num_chunks;
  return GemmShape{256, 256};
}

hipError_t launch_gemm(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b,
                       const uint8_t* bs, int b_layout, int64_t m, int64_t n, int64_t k, uint16_t* c,
                       int64_t ldc, int num_chunks, int first_chunk, int* chunk_done, hipStream_t stream) {
  const GemmShape s = gemm_pick_shape(m, n, num_chunks);
  (void)s;
  return launch_shape<256, 256>(a, as, a_layout, b, bs, b_layout, (int)m, (int)n, (int)k, c, (int)ldc, num_chunks,
                                first_chunk, chunk_done, stream);
}

}  // namespace mxfp8
