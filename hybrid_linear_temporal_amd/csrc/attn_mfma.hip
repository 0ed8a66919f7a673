#include "hlta_device.h"
#include "hlta_launch.h"
namespace hlta {
hipError_t launch_attn_mfma(const AttnParams&, int, hipStream_t) { return hipErrorNotSupported; }
}
