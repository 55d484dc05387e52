// stream_ceiling.hip -- a measurement tool, not part of the library: the
// streaming ceiling of a byte mix.  One kernel reads 4 consecutive elements of
// each of NF fp32, NH 16-bit and NB byte arrays per thread slot and writes
// their sum to NO fp32 arrays, with non-temporal loads and stores: the same
// bytes a workload's kernel must move, with no recurrence.  bench.py times it
// back to back like the library's kernel, over a few launch shapes (U slots
// per thread, grid-strided; B threads per workgroup), and reports the best as
// the practical ceiling of one launch of that size on this machine.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float V4 __attribute__((ext_vector_type(4)));
typedef uint32_t U2 __attribute__((ext_vector_type(2)));

struct Streams {
  const float *f[4];
  const uint16_t *h[2];
  const uint8_t *b[2];
  float *o[2];
};

template <int NF, int NH, int NB, int NO, int U, int B>
__global__ void __launch_bounds__(B) stream_kernel(const Streams S, int64_t n4) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * B;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * B + threadIdx.x + u * stride;
    if (i >= n4) return;
    V4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NF; ++k)
      acc += __builtin_nontemporal_load(reinterpret_cast<const V4 *>(S.f[k]) + i);
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const U2 x = __builtin_nontemporal_load(reinterpret_cast<const U2 *>(S.h[k]) + i);
      acc.x += __uint_as_float(x.x << 16);
      acc.y += __uint_as_float(x.x & 0xffff0000u);
      acc.z += __uint_as_float(x.y << 16);
      acc.w += __uint_as_float(x.y & 0xffff0000u);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const uint32_t x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(S.b[k]) + i);
      acc.x += static_cast<float>(x & 0xffu);
      acc.y += static_cast<float>((x >> 8) & 0xffu);
      acc.z += static_cast<float>((x >> 16) & 0xffu);
      acc.w += static_cast<float>(x >> 24);
    }
#pragma unroll
    for (int k = 0; k < NO; ++k)
      __builtin_nontemporal_store(acc + static_cast<float>(k), reinterpret_cast<V4 *>(S.o[k]) + i);
  }
}

template <int NF, int NH, int NB, int NO, int U, int B>
int launch(const Streams &S, int64_t n4, hipStream_t s) {
  const int64_t per = static_cast<int64_t>(B) * U;
  const int64_t blocks = (n4 + per - 1) / per;
  if (blocks > 0x7fffffff) return -1;
  hipLaunchKernelGGL((stream_kernel<NF, NH, NB, NO, U, B>), dim3(static_cast<unsigned>(blocks)),
                     dim3(B), 0, s, S, n4);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

template <int NF, int NH, int NB, int NO, int U>
int by_block(const Streams &S, int64_t n4, hipStream_t s, int block) {
  switch (block) {
    case 256: return launch<NF, NH, NB, NO, U, 256>(S, n4, s);
    case 512: return launch<NF, NH, NB, NO, U, 512>(S, n4, s);
    case 1024: return launch<NF, NH, NB, NO, U, 1024>(S, n4, s);
    default: return -1;
  }
}

template <int NF, int NH, int NB, int NO>
int by_shape(const Streams &S, int64_t n4, hipStream_t s, int per_thread, int block) {
  switch (per_thread) {
    case 1: return by_block<NF, NH, NB, NO, 1>(S, n4, s, block);
    case 2: return by_block<NF, NH, NB, NO, 2>(S, n4, s, block);
    case 4: return by_block<NF, NH, NB, NO, 4>(S, n4, s, block);
    default: return -1;
  }
}

}  // namespace

// The byte mixes of the library's workloads (fp32 arrays, 16-bit arrays, byte
// arrays, fp32 outputs).  Pointers are device addresses of arrays of `elems`
// elements each (elems a multiple of 4, 16-byte aligned); unused entries are
// ignored.  Returns 0, -1 for an unknown mix or shape, -2 if the launch failed.
extern "C" int stream_ceiling(int nf, int nh, int nb, int no, const float *const *f,
                              const uint16_t *const *h, const uint8_t *const *b, float *const *o,
                              int64_t elems, int per_thread, int block, void *stream) {
  if (elems <= 0 || elems % 4 != 0) return -1;
  Streams S = {};
  for (int k = 0; k < nf && k < 4; ++k) S.f[k] = f[k];
  for (int k = 0; k < nh && k < 2; ++k) S.h[k] = h[k];
  for (int k = 0; k < nb && k < 2; ++k) S.b[k] = b[k];
  for (int k = 0; k < no && k < 2; ++k) S.o[k] = o[k];
  const int64_t n4 = elems / 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mix = nf * 1000 + nh * 100 + nb * 10 + no;
  switch (mix) {
    case 1011: return by_shape<1, 0, 1, 1>(S, n4, s, per_thread, block);  // returns
    case 2022: return by_shape<2, 0, 2, 2>(S, n4, s, per_thread, block);  // GAE
    case 2011: return by_shape<2, 0, 1, 1>(S, n4, s, per_thread, block);  // TD(lambda)
    case 2021: return by_shape<2, 0, 2, 1>(S, n4, s, per_thread, block);  // TD(lambda), truncations
    case 3012: return by_shape<3, 0, 1, 2>(S, n4, s, per_thread, block);  // V-trace
    case 4011: return by_shape<4, 0, 1, 1>(S, n4, s, per_thread, block);  // Retrace
    case 222: return by_shape<0, 2, 2, 2>(S, n4, s, per_thread, block);   // GAE, bf16 inputs
    case 1021: return by_shape<1, 0, 2, 1>(S, n4, s, per_thread, block);  // forward mirrors
    case 1001: return by_shape<1, 0, 0, 1>(S, n4, s, per_thread, block);  // plain copy
    default: return -1;
  }
}
