// hostsim.hip - the GPU lane coder (entropy_coding_02_amd/csrc/lane_coder.h)
// compiled for the host, so CPU tests can compare it with the oracle stream
// by stream before any kernel runs.  Test infrastructure only.
#include <stdint.h>

#include "../../entropy_coding_02_amd/csrc/lane_coder.h"

extern "C" {

// Encode one stream into `slot` (>= round_up(2C+16, 16) bytes); returns its length.
int64_t hostsim_encode_stream(const uint8_t *q, int32_t C, int32_t A, const uint16_t *cdf_rows,
                              uint8_t *slot)
{
    EncState e;
    enc_init(e);
    SlotOut out{(uint32_t *)slot};
    for (int32_t c = 0; c < C; ++c) enc_symbol(e, cdf_rows + (int64_t)c * A, (uint32_t)A, q[c], out);
    return enc_finish(e, out);
}

// Decode the stream at [off, off+len) of a buffer of `cap` bytes; returns the corrupt flag.
int hostsim_decode_stream(const uint8_t *buf, int64_t cap, int64_t off, int64_t len, int32_t C,
                          int32_t A, const uint16_t *cdf_rows, uint8_t *q)
{
    StreamIn in;
    in.init(buf, (uint64_t)off, (uint64_t)len, (uint64_t)cap);
    DecState d;
    dec_init(d, in);
    uint32_t bad = 0, step0 = dec_step0((uint32_t)A);
    for (int32_t c = 0; c < C; ++c)
        q[c] = (uint8_t)dec_symbol(d, cdf_rows + (int64_t)c * A, (uint32_t)A, step0, in, &bad);
    return (int)bad;
}

}  // extern "C"
