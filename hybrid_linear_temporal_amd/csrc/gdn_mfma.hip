#include "hlta_device.h"
#include "hlta_launch.h"
namespace hlta {
hipError_t launch_gdn_mfma(const GdnParams&, int, hipStream_t) { return hipErrorNotSupported; }
}
