// gdr_kernels.h -- host-callable launchers of the libgdr kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// Optional timing of one launch: events recorded by the runtime at the
// kernel's start and end (hipExtLaunchKernelGGL).  Null events: no timing.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

void launch_table(const int32_t* cu, int32_t N, int32_t T, int32_t nslots, int4* table,
                  int32_t* choff, hipStream_t stream, LaunchEvents ev = {});

// Intra-chunk products for chunk slots [slot0, slot0 + nseg) of every value head;
// also writes exp(total gate of the chunk) to gam[slot][head].
template <typename Tin>
hipError_t launch_intra(const Tin* q, const Tin* k, const Tin* v, const float* g, const float* beta,
                        const int4* table, int32_t Nqk, int32_t Nv, int32_t slot0, int32_t nseg,
                        float scale, int norm, Tin* inter, float* gam, hipStream_t stream,
                        LaunchEvents ev = {});

// Chunk-serial state pass over chunk slots [slot0, slot0 + nseg).  `discard` is
// 256 bytes of scratch that absorbs the stores of rows past a chunk's end.
template <typename Tin>
void launch_inter(const Tin* inter, const int4* table, const int32_t* choff, const float* gam,
                  const float* state_in, float* carry, float* state_out, int32_t N, int32_t Nv,
                  int32_t slot0, int32_t nseg, bool first_segment, Tin* out, Tin* discard,
                  hipStream_t stream, LaunchEvents ev = {});

template <typename Tin>
void launch_decode(const Tin* q, const Tin* k, const Tin* v, const float* g, const float* beta,
                   const float* state_in, float* state_out, int32_t N, int32_t Nqk, int32_t Nv,
                   float scale, int norm, Tin* out, hipStream_t stream, LaunchEvents ev = {});

}  // namespace gdr
