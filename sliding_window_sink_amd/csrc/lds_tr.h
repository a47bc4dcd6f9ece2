// lds_tr.h -- transposing LDS reads of gfx950 (ds_read_b64_tr_b16) for MFMA operands.
//
// Layout of the instruction (measured on the GPU): within each group of 16 lanes,
// lane s supplies the address of 4 consecutive 16-bit elements, and lane j
// receives element (j % 4) of the chunks supplied by lanes 4e + j/4, e = 0..3.
// So if lanes 4e .. 4e+3 of a group point at the same row (e.g. a key) and at 4
// consecutive 4-element column chunks, lane j ends up holding column
// (chunk(j/4) + j%4) of the 4 rows e = 0..3: a row-major tile is read as its
// transpose, 4 rows per load.  Two loads fill an 8-element MFMA operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

typedef short lds_tr_s4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_tr16(const uint16_t *p) {
    const lds_tr_s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) lds_tr_s4 *)(const_cast<uint16_t *>(p)));
    return __builtin_bit_cast(uint2, r);
}

}  // namespace sinkattn
