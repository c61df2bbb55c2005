// mb_stream.hip -- the streaming ceiling the benchmark measures each fused op
// against (libmb_stream.so; benchmark support, not part of the library's ABI).
//
// A fused epilogue moves each of its tensors once; what limits it is how fast
// the GPU streams that mix of reads and writes. This kernel moves exactly the
// bytes of an op -- the same tensors, row pitches, 16- or 8-byte pieces per
// lane, column-strip tiling (a block of 4 waves, each wave a strip of 64
// lanes walking rows) and non-temporal loads and stores as the op's kernel --
// and does no arithmetic beyond an xor that keeps every load live. The
// benchmark sweeps the launch shape (blocks, rows in flight) and the store
// form (global non-temporal, or buffer non-temporal at system scope) and
// takes the fastest, so the ceiling is the best this tiling streams that mix.
#include <stdint.h>

#include "mb_device.hpp"

namespace {

using namespace mb;

constexpr int kMaxIn = 3, kMaxOut = 2;

struct Bufs {
  const char* in[kMaxIn];
  int64_t in_pitch[kMaxIn];
  char* out[kMaxOut];
  int64_t out_pitch[kMaxOut];
  int64_t rows;
  int lanes;
};

// LD < 0: global non-temporal load at `at`; else a buffer load with cache
// policy LD at byte `off` of the wave-uniform row `row` (at == row + off).
template <bool EIGHT, int LD> __device__ __forceinline__ u32x4 load_piece(const char* at, const char* row, uint32_t off) {
  if constexpr (EIGHT) {
    u32x2 v;
    if constexpr (LD < 0) {
      v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(at));
    } else {
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row), 0, 0x7fffffff, 0x00020000);
      v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, LD);
    }
    const unsigned a = v.x, b = v.y;
    return u32x4{a, b, 0u, 0u};
  } else {
    return ld_row<LD>(at, row, off);
  }
}

// ST < 0: global non-temporal store at `at`; else a buffer store with cache
// policy ST at byte `off` of the wave-uniform row `row` (at == row + off).
template <bool EIGHT, int ST> __device__ __forceinline__ void store_piece(char* at, char* row, uint32_t off, u32x4 v) {
  if constexpr (EIGHT) {
    // fold the upper half in, so that a 16-byte input feeding an 8-byte
    // output is still loaded whole
    const unsigned a = v.x ^ v.z, b = v.y ^ v.w;
    const u32x2 w = {a, b};
    if constexpr (ST < 0)
      __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(at));
    else
      st_buf<ST>(row, off, w);
  } else {
    if constexpr (ST < 0)
      st_stream(at, v);
    else
      st_buf<ST>(row, off, v);
  }
}

// NR inputs and NW outputs; bit i of R8 / W8: input / output i moves 8-byte
// pieces per lane (else 16). U rows in flight per wave. LD, ST: load and
// store forms (-1 global non-temporal, else the buffer cache policy).
template <int NR, int NW, unsigned R8, unsigned W8, int U, int LD, int ST>
__global__ __launch_bounds__(kThreads) void stream_kernel(Bufs b) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_index<(ST >= 0 || LD >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  if (cv >= b.lanes) return;
  const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
  for (int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave; t < b.rows; t += U * S) {
    u32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc[u] = u32x4{0u, 0u, 0u, 0u};
      const int64_t tt = t + u * S;
      if (tt < b.rows) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const bool eight = (R8 >> i) & 1u;
          const uint32_t off = static_cast<uint32_t>(cv) * (eight ? 8u : 16u);
          const char* row = b.in[i] + tt * b.in_pitch[i];
          acc[u] ^= eight ? load_piece<true, LD>(row + off, row, off) : load_piece<false, LD>(row + off, row, off);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tt = t + u * S;
      if (tt >= b.rows) break;
#pragma unroll
      for (int o = 0; o < NW; ++o) {
        const bool eight = (W8 >> o) & 1u;
        const uint32_t off = static_cast<uint32_t>(cv) * (eight ? 8u : 16u);
        char* row = b.out[o] + tt * b.out_pitch[o];
        const u32x4 v = acc[u] ^ u32x4{static_cast<unsigned>(o), 0u, 0u, 0u};
        if (eight)
          store_piece<true, ST>(row + off, row, off, v);
        else
          store_piece<false, ST>(row + off, row, off, v);
      }
    }
  }
}

template <int NR, int NW, unsigned R8, unsigned W8, int U, int LD, int ST>
hipError_t launch_one(const Bufs& b, int G, hipStream_t s) {
  const int strips = (b.lanes + kStrip - 1) / kStrip;
  hipLaunchKernelGGL((stream_kernel<NR, NW, R8, W8, U, LD, ST>), tile_grid(strips, G), dim3(kThreads), 0, s, b);
  return hipGetLastError();
}

// io bit 0: buffer non-temporal stores at system scope (else global
// non-temporal); bit 1: buffer non-temporal loads (else global non-temporal)
template <int NR, int NW, unsigned R8, unsigned W8, int U>
hipError_t launch_io(const Bufs& b, int G, int io, hipStream_t s) {
  switch (io) {
    case 0: return launch_one<NR, NW, R8, W8, U, -1, -1>(b, G, s);
    case 1: return launch_one<NR, NW, R8, W8, U, -1, 18>(b, G, s);
    case 2: return launch_one<NR, NW, R8, W8, U, 2, -1>(b, G, s);
    case 3: return launch_one<NR, NW, R8, W8, U, 2, 18>(b, G, s);
  }
  return hipErrorInvalidValue;
}

template <int NR, int NW, unsigned R8, unsigned W8>
hipError_t launch_u(const Bufs& b, int G, int U, int io, hipStream_t s) {
  switch (U) {
    case 1: return launch_io<NR, NW, R8, W8, 1>(b, G, io, s);
    case 2: return launch_io<NR, NW, R8, W8, 2>(b, G, io, s);
    case 4: return launch_io<NR, NW, R8, W8, 4>(b, G, io, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

extern "C" {

// One streaming pass: rows x lanes pieces from each of n_in inputs, the xor of
// them to each of n_out outputs. in8 / out8: bit i set when buffer i moves
// 8-byte pieces (else 16-byte). Supported mixes: 1-3 inputs and 1-2 outputs of
// 16-byte pieces; (8-byte, 16-byte) inputs to one 8-byte output; one 8-byte
// input to (8-byte, 16-byte) outputs. blocks: grid size to aim for (row groups
// = blocks / strips, at least 1, at most ceil(rows / 4) and 65535);
// rows_in_flight 1, 2 or 4; io bit 0: stores through a buffer descriptor,
// non-temporal at system scope (else global non-temporal stores), bit 1:
// loads through a buffer descriptor, non-temporal (else global non-temporal
// loads). Pointers are device pointers, 16-byte aligned,
// each buffer holding rows * pitch bytes. Returns 0, or -1 for an unsupported
// mix or shape, or the HIP error of the launch.
int mbs_stream(const void* const* in, const int64_t* in_pitch, int n_in, unsigned in8, void* const* out,
               const int64_t* out_pitch, int n_out, unsigned out8, int64_t rows, int lanes, int blocks,
               int rows_in_flight, int io, hipStream_t s) {
  if (n_in < 1 || n_in > kMaxIn || n_out < 1 || n_out > kMaxOut || rows <= 0 || lanes <= 0) return -1;
  if (io < 0 || io > 3) return -1;
  const int strips = (lanes + kStrip - 1) / kStrip;
  if (strips > 65535) return -1;
  Bufs b{};
  for (int i = 0; i < n_in; ++i) {
    b.in[i] = static_cast<const char*>(in[i]);
    b.in_pitch[i] = in_pitch[i];
  }
  for (int o = 0; o < n_out; ++o) {
    b.out[o] = static_cast<char*>(out[o]);
    b.out_pitch[o] = out_pitch[o];
  }
  b.rows = rows;
  b.lanes = lanes;
  int64_t G = blocks / strips;
  if (G < 1) G = 1;
  const int64_t most = (rows + kWaves - 1) / kWaves;
  if (G > most) G = most;
  if (G > 65535) G = 65535;
  const int g = static_cast<int>(G);
  if (in8 == 0 && out8 == 0) {
    if (n_in == 1 && n_out == 1) return launch_u<1, 1, 0, 0>(b, g, rows_in_flight, io, s);
    if (n_in == 2 && n_out == 1) return launch_u<2, 1, 0, 0>(b, g, rows_in_flight, io, s);
    if (n_in == 3 && n_out == 1) return launch_u<3, 1, 0, 0>(b, g, rows_in_flight, io, s);
    if (n_in == 1 && n_out == 2) return launch_u<1, 2, 0, 0>(b, g, rows_in_flight, io, s);
    if (n_in == 2 && n_out == 2) return launch_u<2, 2, 0, 0>(b, g, rows_in_flight, io, s);
    if (n_in == 3 && n_out == 2) return launch_u<3, 2, 0, 0>(b, g, rows_in_flight, io, s);
  }
  if (n_in == 2 && n_out == 1 && in8 == 1u && out8 == 1u)
    return launch_u<2, 1, 1u, 1u>(b, g, rows_in_flight, io, s);
  if (n_in == 1 && n_out == 2 && in8 == 1u && out8 == 1u)
    return launch_u<1, 2, 1u, 1u>(b, g, rows_in_flight, io, s);
  return -1;
}

}  // extern "C"
